"""The no-allocation backward (fa_bwd_noalloc, through the C ABI) against fa_bwd with a caller
workspace: calls in a row, the second on a smaller problem, the third on a stream the test creates
(the scratch is looked up through the stream's device), each bit-identical to fa_bwd and within
the gradient bar of the oracle on one head; a problem beyond the scratch is refused."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from inputs import randn_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_numerical_stability_amd as fa_mod
    torch.zeros(1, device=DEV)
    return fa_mod


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_no_alloc_backward_matches_workspace_backward(fa):
    from precision_numerical_stability_amd import _ffi
    lib = _ffi.load_library()
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream(device=DEV)  # default priority
    # the second problem is smaller: the scratch keeps the first call's delta beyond its rows
    cases = ((2, 4, 1000, 128, True, 3100, False), (1, 3, 333, 64, False, 3101, False),
             (1, 2, 700, 128, True, 3102, True))
    for (B, H, N, d, causal, seed, on_side) in cases:
        print(f"[case] noalloc B={B} H={H} N={N} d={d} causal={causal} side_stream={on_side}", flush=True)
        t = randn_inputs(B, H, N, d, seed=seed)
        g = {k: v.to(DEV) for k, v in t.items()}
        scale = d ** -0.5
        o, lse = fa.forward(g["q"], g["k"], g["v"], causal, scale, 1.25, 1)
        ref = [torch.empty_like(g["q"]) for _ in range(3)]
        delta = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
        fa.fa_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], *ref, delta, causal, scale)
        got = [torch.full_like(g["q"], 7.0) for _ in range(3)]
        stream = side if on_side else main
        if on_side:
            side.wait_stream(main)  # the inputs and outputs were written on the main stream
        rc = lib.fa_bwd_noalloc(_p(g["q"]), _p(g["k"]), _p(g["v"]), _p(o), _p(lse), _p(g["do"]),
                                *(_p(x) for x in got), B, H, N, d, int(causal), scale, 1.25, 1,
                                ctypes.c_void_p(stream.cuda_stream))
        assert rc == 0, fa.fa_status_str(rc)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"{name} differs from fa_bwd"
        x = {k: v[0, 0].to(torch.float64).numpy() for k, v in t.items()}
        br = oracle.backward(x["q"], x["k"], x["v"], x["do"], causal, scale)
        for name, a, r in zip(("dq", "dk", "dv"), got, (br.dq, br.dk, br.dv)):
            err = np.abs(a[0, 0].float().cpu().numpy() - r).max()
            assert err <= 3e-2 * np.abs(r).max() + 1e-5, f"{name}: {err:.3e}"
    # beyond the scratch: refused before anything is launched
    big = lib.fa_bwd_noalloc_max_rows() + 1
    assert lib.fa_bwd_noalloc(*([_p(g["q"])] * 9), 1, 1, big, 64, 0, 0.125, 1.25, 1, None) == fa.FA_ERR_SCRATCH

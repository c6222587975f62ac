"""GPU parity of the fp16 element type (fa_fwd_elem / fa_bwd_elem with FA_ELEM_F16) against the
fp64 oracle on the same seeded fp16 inputs.

The same bars as for bf16: O within 1e-2 + 1e-2 |O_ref| elementwise; LSE within 1e-3 absolute;
dQ, dK, dV within 3e-2 of each tensor's max |ref|; repeat counts bit-exact; exact-1.0 counts
bit-exact against the oracle's key-block replay with P^ rounded to binary16; no NaN or Inf.

Range: binary16 tops out at 65504, which e^12 already exceeds ([FA-backward] §3.1), so an
unshifted exponential of a score of 12 or more would overflow.  The kernels only ever take
exp(S - m) with m at least the running maximum (P^ <= 1), so scores far above 12 stay finite; the
tests below put row maxima at 12, 40 and, with sigma = 3 inputs, up to ~46.
"""
import numpy as np
import pytest
import torch

import oracle
from inputs import CONFIGS, make_inputs, randn_inputs, rect_inputs, grid_inputs
from test_parity_gpu import DEV, BETA, _say, _to_dev, check_o, check_lse, check_grad

pytestmark = pytest.mark.gpu

F16 = torch.float16


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_numerical_stability_amd as fa_mod
    from precision_numerical_stability_amd import _ffi
    torch.zeros(1, device=DEV)
    assert len(_ffi.hip_runtimes_mapped()) == 1, _ffi.hip_runtimes_mapped()
    return fa_mod


def run16(fa, t, causal, scale, mode, bwd=True):
    """Forward (with counts) and backward through the fp16 entry points; numpy results."""
    g = _to_dev(t)
    assert g["q"].dtype == F16
    o, lse, dup, ones = fa.forward(g["q"], g["k"], g["v"], causal, scale, BETA, mode, stats=True)
    out = {"o": o, "lse": lse, "dup": dup, "ones": ones}
    if bwd:
        dq, dk, dv = fa.backward(g["q"], g["k"], g["v"], o, lse, g["do"], causal, scale)
        assert dq.dtype == F16 and dk.dtype == F16 and dv.dtype == F16
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert o.dtype == F16
    res = {k_: (v_.float() if v_.dtype == F16 else v_).cpu().numpy() for k_, v_ in out.items()}
    for k_ in ("o", "dup", "ones", "dq", "dk", "dv"):
        if k_ in res:
            assert np.all(np.isfinite(res[k_])), f"non-finite values in {k_}"
    return res


def check16(res, t, b, h, causal, scale, mode, grads=True, counts_exact=False, bc=None):
    x = {k_: v_[b, h].to(torch.float64).numpy() for k_, v_ in t.items()}
    fr = oracle.forward(x["q"], x["k"], x["v"], causal, scale, BETA, mode, elem="f16")
    check_o(res["o"][b, h], fr.o, f"O[{b},{h}]")
    empty = fr.lse == -np.inf
    lse = res["lse"][b, h]
    assert np.array_equal(lse == -np.inf, empty)
    if (~empty).any():
        check_lse(lse[~empty], fr.lse[~empty])
    if counts_exact:
        assert np.array_equal(res["dup"][b, h], fr.rs), f"dupcnt[{b},{h}] differs"
        want = oracle.tiled_ones(x["q"], x["k"], causal, scale, BETA, mode, bc=bc, elem="f16")
        diff = np.nonzero(res["ones"][b, h] != want)[0]
        assert diff.size == 0, f"ones[{b},{h}] differs at rows {diff[:10]}"
    if grads:
        br = oracle.backward(x["q"], x["k"], x["v"], x["do"], causal, scale, o=fr.o, lse=fr.lse)
        for name, ref in (("dq", br.dq), ("dk", br.dk), ("dv", br.dv)):
            check_grad(res[name][b, h], ref, f"{name}[{b},{h}]")
    return fr


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_f16_tiny_duplicates(fa, mode):
    cfg = CONFIGS[1]
    _say("f16-config1", mode)
    t = make_inputs(cfg, dtype=F16)
    res = run16(fa, t, cfg.causal, cfg.scale, mode)
    check16(res, t, 0, 0, cfg.causal, cfg.scale, mode, counts_exact=True,
            bc=fa.fa_fwd_kv_block(cfg.d, cfg.causal))
    assert np.all(res["dup"][0, 0, :8] == 2)
    assert np.all(res["ones"][0, 0, :8] == (2 if mode == 0 else 0))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1, 2])
@pytest.mark.parametrize("nq,nk", [(333, 333), (37, 300), (300, 37), (256, 513)])
def test_f16_shapes(fa, d, causal, nq, nk):
    _say("f16-shape", d, causal, nq, nk)
    t = rect_inputs(2, 2, nq, nk, d, seed=1600 + nq + 3 * nk + d + causal, dtype=F16)
    scale = d ** -0.5
    res = run16(fa, t, causal, scale, 1)
    for b, h in ((0, 0), (1, 1)):
        fr = check16(res, t, b, h, causal, scale, 1)
        empty = fr.lse == -np.inf
        assert np.all(res["o"][b, h][empty] == 0) and np.all(res["dq"][b, h][empty] == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_f16_grid_counts(fa, causal):
    """Grid inputs: every dot product is exact in fp32, so repeat counts and exact-1.0 counts are
    bit-exact in every mode."""
    _say("f16-grid", causal)
    t = grid_inputs(1, 2, 320, 128, seed=1677, dtype=F16)
    scale = 128 ** -0.5
    bc = fa.fa_fwd_kv_block(128, causal)
    for mode in (0, 1, 2):
        res = run16(fa, t, causal, scale, mode, bwd=(mode == 1))
        for h in range(2):
            check16(res, t, 0, h, causal, scale, mode, grads=(mode == 1), counts_exact=True, bc=bc)


def test_f16_sink_large_logits(fa):
    """sigma = 3 queries and keys with an attention-sink key (the GPT-2-medium-like workload, 2 of
    its heads): row maxima far above ln(65504) ~ 11.09, where an unshifted binary16 exponential
    would already be inf."""
    cfg = CONFIGS[3]
    _say("f16-sink")
    t = make_inputs(cfg, dtype=F16, B=1, H=2)
    res = run16(fa, t, cfg.causal, cfg.scale, 1)
    for h in range(2):
        fr = check16(res, t, 0, h, cfg.causal, cfg.scale, 1)
        big = fr.rm > 12.0
        assert big.sum() > 100, "the workload should put many row maxima above 12"
        assert np.all(np.isinf(oracle.fp16_round(np.exp(fr.rm[big]))))


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("top", [12.0, 40.0])
def test_f16_constructed_maxima_at_and_above_e12(fa, mode, top):
    """Rows whose maximum score is exactly `top` (12 or 40), attained twice (keys 5 and 9):
    q_i = k_5 = k_9 = c on the first n coordinates, so S = scale n c^2 = top exactly in fp32.
    Mode 0 leaves P^ = 1.0 at both maxima (counted by ones); modes 1 and 2 shift the row to
    beta * top, so P^ = e^{-(beta - 1) top} there and no exact 1.0 remains."""
    _say("f16-e12", mode, top)
    N, d, scale = 128, 64, 0.125
    c, n = (2.0, 24) if top == 12.0 else (4.0, 20)  # 0.125 * 24 * 4 = 12, 0.125 * 20 * 16 = 40
    gen = torch.Generator().manual_seed(1612 + int(top))
    q = (0.25 * torch.randn(1, 1, N, d, generator=gen))
    k = (0.25 * torch.randn(1, 1, N, d, generator=gen))
    v = torch.randn(1, 1, N, d, generator=gen)
    do = torch.randn(1, 1, N, d, generator=gen)
    row = torch.zeros(d)
    row[:n] = c
    for j in (5, 9):
        k[0, 0, j] = row
    rows = list(range(10, 30))
    for i in rows:
        q[0, 0, i] = row
    t = {n_: x_.to(F16) for n_, x_ in (("q", q), ("k", k), ("v", v), ("do", do))}
    res = run16(fa, t, False, scale, mode)
    fr = check16(res, t, 0, 0, False, scale, mode, counts_exact=True, bc=fa.fa_fwd_kv_block(d, False))
    assert np.all(fr.rm[rows] == top) and np.all(fr.rs[rows] == 2)
    assert np.isinf(oracle.fp16_round(np.exp(top)))  # an unshifted exponential would overflow
    assert np.all(res["ones"][0, 0, rows] == (2 if mode == 0 else 0))


def test_f16_more_accurate_than_bf16(fa):
    """The same fp32 draws rounded to fp16 and to bf16: against the oracle on its own inputs, the
    fp16 path's O error is well below the bf16 path's (binary16 keeps 3 more significant bits for
    P^ and for O)."""
    _say("f16-vs-bf16")
    errs = {}
    scale = 128 ** -0.5
    for dt in (torch.bfloat16, F16):
        t = randn_inputs(1, 2, 512, 128, seed=1650, dtype=dt)
        g = _to_dev(t)
        o, _ = fa.forward(g["q"], g["k"], g["v"], True, scale, BETA, 1)
        o = o.float().cpu().numpy()
        e = 0.0
        for h in range(2):
            x = {k_: v_[0, h].to(torch.float64).numpy() for k_, v_ in t.items()}
            fr = oracle.forward(x["q"], x["k"], x["v"], True, scale, BETA, 1)
            e = max(e, np.abs(o[0, h] - fr.o).max())
        errs[dt] = e
    assert errs[F16] < 0.5 * errs[torch.bfloat16], errs


def test_f16_llama_head(fa):
    """One head of the LLaMA-7B-shaped workload (N = 8192, d = 128, causal) in fp16, mode 1,
    forward and backward."""
    cfg = CONFIGS[4]
    _say("f16-llama")
    t = make_inputs(cfg, dtype=F16, H=1)
    res = run16(fa, t, cfg.causal, cfg.scale, 1)
    check16(res, t, 0, 0, cfg.causal, cfg.scale, 1)


def test_f16_autograd_wrapper(fa):
    _say("f16-autograd")
    t = _to_dev(make_inputs(2, dtype=F16, B=1, H=2, N=256))
    q, k, v = (t[n_].clone().requires_grad_(True) for n_ in ("q", "k", "v"))
    o = fa.attention(q, k, v, causal=True, scale=0.125)
    assert o.dtype == F16
    o.backward(t["do"])
    o2, lse2 = fa.forward(t["q"], t["k"], t["v"], True, 0.125, BETA, fa.TIE_RULE)
    dq2, dk2, dv2 = fa.backward(t["q"], t["k"], t["v"], o2, lse2, t["do"], True, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    for a_, b_ in ((q.grad, dq2), (k.grad, dk2), (v.grad, dv2)):
        assert a_.dtype == F16 and torch.equal(a_, b_)


def test_f16_bf16_entry_points_agree_on_bf16(fa):
    """fa_fwd_elem / fa_bwd_elem with FA_ELEM_BF16 are the bf16 entry points, bit for bit."""
    _say("elem-bf16")
    g = _to_dev(rect_inputs(1, 2, 200, 300, 64, seed=1690))
    o1, lse1 = torch.empty_like(g["q"]), torch.empty((1, 2, 200), device=DEV)
    fa.fa_fwd_qk(g["q"], g["k"], g["v"], o1, lse1, None, None, None, None, 2, 0.125, BETA, 1)
    o2, lse2 = torch.empty_like(g["q"]), torch.empty((1, 2, 200), device=DEV)
    fa.fa_fwd_elem(g["q"], g["k"], g["v"], o2, lse2, None, None, None, None, 2, 0.125, BETA, 1)
    grads = []
    for fn, o, lse in ((fa.fa_bwd_qk, o1, lse1), (fa.fa_bwd_elem, o2, lse2)):
        dq, dk, dv = torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"])
        fn(g["q"], g["k"], g["v"], o, lse, g["do"], dq, dk, dv, torch.empty_like(lse), 2, 0.125)
        grads.append((dq, dk, dv))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2)
    for a_, b_ in zip(*grads):
        assert torch.equal(a_, b_)


def test_f16_rejects_mixed_element_types(fa):
    q = torch.zeros((1, 1, 128, 64), dtype=F16, device=DEV)
    k = torch.zeros((1, 1, 128, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        fa.forward(q, k, k, False, 0.125)


@pytest.mark.parametrize("compensated", [False, True])
@pytest.mark.parametrize("causal,nq,nk", [(0, 256, 256), (1, 333, 333), (2, 300, 100)])
def test_f16_monitors_and_compensated_sum(fa, compensated, causal, nq, nk):
    """The diagnostics variant in fp16: per-row score range (smin, smax), repeat counts and the
    compensated row sum, against the oracle; the gradients from its LSE."""
    _say("f16-monitor", compensated, causal, nq, nk)
    t = rect_inputs(1, 2, nq, nk, 64, seed=1700 + nq + nk + causal, dtype=F16)
    g = _to_dev(t)
    scale = 0.125
    o, lse, dup, ones, smin, smax = fa.forward(g["q"], g["k"], g["v"], causal, scale, BETA, 2,
                                               stats=True, monitor=True,
                                               compensated_sum=compensated)
    dq, dk, dv = fa.backward(g["q"], g["k"], g["v"], o, lse, g["do"], causal, scale)
    torch.cuda.synchronize()
    res = {"o": o.float().cpu().numpy(), "lse": lse.cpu().numpy(), "dup": dup.cpu().numpy(),
           "ones": ones.cpu().numpy(), "dq": dq.float().cpu().numpy(),
           "dk": dk.float().cpu().numpy(), "dv": dv.float().cpu().numpy()}
    for h in range(2):
        fr = check16(res, t, 0, h, causal, scale, 2)
        empty = fr.lse == -np.inf
        got_min, got_max = smin[0, h].cpu().numpy(), smax[0, h].cpu().numpy()
        assert np.all(got_min[empty] == np.inf) and np.all(got_max[empty] == -np.inf)
        np.testing.assert_allclose(got_min[~empty], fr.smin[~empty], rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(got_max[~empty], fr.rm[~empty], rtol=1e-5, atol=1e-5)
        # Mode 2 shifts every row off its maximum, so no P^ rounds to 1.0 unless the maximum is
        # within ~2^-12 of 0 (then e^{-(beta - 1) rm} or e^{rm} rounds to 1 in binary16).
        away = ~empty & (np.abs(fr.rm) > 1e-2)
        assert away.sum() > 0.9 * (~empty).sum() and np.all(res["ones"][0, h][away] == 0)

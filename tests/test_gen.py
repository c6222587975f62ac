"""Seeded input generators: determinism and the constructions each workload calls for."""
import numpy as np
import torch

from inputs import CONFIGS, make_inputs, tensor_digest
from inputs.gen import GRID_VALUES


def test_deterministic_and_seed_sensitive():
    a = make_inputs(2, B=1, H=2, N=256)
    b = make_inputs(2, B=1, H=2, N=256)
    c = make_inputs(2, B=1, H=2, N=256, seed=7)
    for name in ("q", "k", "v", "do"):
        assert tensor_digest(a[name]) == tensor_digest(b[name])
        assert tensor_digest(a[name]) != tensor_digest(c[name])
        assert a[name].dtype == torch.bfloat16 and a[name].is_contiguous()


def test_config1_duplicates():
    t = make_inputs(1)
    assert t["q"].shape == (1, 1, 128, 64)
    assert torch.equal(t["k"][0, 0, 17], t["k"][0, 0, 3])
    for i in range(8):
        assert torch.equal(t["q"][0, 0, i], t["k"][0, 0, 3])


def test_config3_sink_and_sigma():
    t = make_inputs(3, B=2, H=2, N=512)
    q = t["q"].to(torch.float64)
    assert 2.5 < q.std().item() < 3.5
    for b in range(2):
        for h in range(2):
            u = q[b, h].mean(dim=0)
            u = u / u.norm()
            k0 = t["k"][b, h, 0].to(torch.float64)
            assert abs(k0.norm().item() - 4.0) < 0.05
            assert torch.dot(k0 / k0.norm(), u).item() > 0.999


def test_config5_grid_values():
    t = make_inputs(5, H=1, N=1024)
    for name in ("q", "k"):
        vals = set(np.unique(t[name].to(torch.float32).numpy()).tolist())
        assert vals <= set(GRID_VALUES)
    assert t["v"].to(torch.float32).std().item() > 0.9


def test_config_table():
    assert CONFIGS[4].B == 1 and CONFIGS[4].H == 32 and CONFIGS[4].N == 8192 and CONFIGS[4].d == 128
    assert CONFIGS[4].causal and abs(CONFIGS[4].scale - 128 ** -0.5) < 1e-8
    assert CONFIGS[5].N == 16384 and CONFIGS[5].kind == "grid"
    assert not CONFIGS[1].causal and CONFIGS[1].scale == 0.125


def test_rect_inputs_shapes_and_determinism():
    from inputs import rect_inputs
    a = rect_inputs(2, 3, 70, 300, 64, seed=5)
    b = rect_inputs(2, 3, 70, 300, 64, seed=5)
    assert a["q"].shape == (2, 3, 70, 64) and a["do"].shape == (2, 3, 70, 64)
    assert a["k"].shape == (2, 3, 300, 64) and a["v"].shape == (2, 3, 300, 64)
    for name in a:
        assert torch.equal(a[name], b[name]) and a[name].dtype == torch.bfloat16
    g = rect_inputs(1, 1, 8, 16, 128, seed=5, grid=True)
    vals = set(g["q"].float().unique().tolist()) | set(g["k"].float().unique().tolist())
    assert vals <= set(GRID_VALUES)

"""Pins for the fp64 oracle: each check ties it to something other than its own code.

Pins used: brute force with scalar Python loops, the pages' printed numbers and closed forms,
torch's bf16 cast, finite differences, exact integer arithmetic, and invariants of the gradient.
None of these tests touches a GPU.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from inputs import make_inputs, grid_inputs, rect_inputs, tied_maxima_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BETA = 1.25


def _np(t):
    return t.to(torch.float64).numpy()


def _head(t, b=0, h=0):
    return {k: _np(v[b, h]) for k, v in t.items()}


def _scores_row(values, scale=1.0):
    """Q and K with one query row whose scaled scores are exactly `values` (d = 2)."""
    n = len(values)
    q = np.zeros((1, 2))
    q[0, 0] = 1.0
    k = np.zeros((n, 2))
    k[:, 0] = np.asarray(values, dtype=np.float64) / scale
    return q, k


# ----------------------------------------------------------------------------------------------
# bf16 rounding (the format of the BF16 article, §1; RNE per its §2.2)


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        rng.uniform(0.98, 1.0, 20000).astype(np.float32),
        np.exp(-rng.uniform(0, 30, 20000)).astype(np.float32),
    ])
    # exact halfway cases between adjacent bf16 values, both parities
    base = np.array([1.0, 1.0078125, 0.99609375, 3.0, 0.5], dtype=np.float32)
    ulp = np.array([2 ** -7, 2 ** -7, 2 ** -8, 2 ** -6, 2 ** -9], dtype=np.float32)
    x = np.concatenate([x, base + ulp / 2, base - ulp / 4 * 0 - ulp / 2])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_round_threshold_below_one():
    # the largest value below 1 that still rounds to 1.0: 1 - 2^-9 (a tie, rounds to even = 1.0)
    assert oracle.bf16_round(1 - 2 ** -9) == 1.0
    assert oracle.bf16_round(np.nextafter(1 - 2 ** -9, 0)) == 1 - 2 ** -8


def test_fp16_round_matches_numpy_and_torch():
    rng = np.random.default_rng(8)
    x = np.concatenate([
        rng.standard_normal(20000) * 300.0,
        rng.uniform(0.998, 1.002, 20000),
        np.exp(-rng.uniform(0, 20, 20000)),  # down through the subnormal range
        np.exp(rng.uniform(10, 11.2, 2000)),  # up to and past the overflow threshold
        -np.exp(rng.uniform(10, 11.2, 2000)),
    ])
    # exact ties: halfway between neighbours, including the subnormal and overflow boundaries
    ties = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 1 - 2 ** -12, 2 ** -25, 3 * 2 ** -25,
                     65520.0, 65488.0, -65520.0, 2 ** -14 + 2 ** -25])
    x = np.concatenate([x, ties])
    got = oracle.fp16_round(x)
    ref = x.astype(np.float16).astype(np.float64)  # numpy rounds float64 -> binary16 directly
    assert np.array_equal(got, ref, equal_nan=False)
    x32 = x.astype(np.float32)  # torch's cast from values exact in fp32 (no double rounding)
    ref32 = torch.from_numpy(x32).to(torch.float16).to(torch.float64).numpy()
    assert np.array_equal(oracle.fp16_round(x32.astype(np.float64)), ref32)


def test_fp16_round_pages_range():
    g = json.load(open(os.path.join(GOLDEN, "pages_numbers.json")))
    assert oracle.fp16_round(g["fp16_max"]["value"]) == 65504.0
    assert oracle.fp16_round(65519.99) == 65504.0 and oracle.fp16_round(65520.0) == np.inf
    assert oracle.fp16_round(math.exp(11)) == 59872.0  # e^11 survives (to the nearest 32)
    assert oracle.fp16_round(math.exp(12)) == np.inf  # e^12 overflows
    assert oracle.fp16_round(g["fp16_min_positive"]["value"]) == 2.0 ** -24
    assert oracle.fp16_round(2.0 ** -25) == 0.0 and oracle.fp16_round(1.5 * 2 ** -25) == 2.0 ** -24
    lo, hi = ONE_WINDOW["f16"]
    assert oracle.fp16_round(lo) == 1.0 and oracle.fp16_round(np.nextafter(lo, 0)) < 1.0
    assert oracle.fp16_round(hi) == 1.0 and oracle.fp16_round(np.nextafter(hi, 2)) > 1.0
    lo, hi = ONE_WINDOW["bf16"]
    assert oracle.bf16_round(lo) == 1.0 and oracle.bf16_round(hi) == 1.0
    assert oracle.bf16_round(np.nextafter(hi, 2)) > 1.0


def test_shifted_fp16_softmax_never_overflows():
    """A softmax whose exponentials are rounded to fp16 overflows for scores above ln 65504 ~ 11.09
    unless the row maximum (or the stabilised shift) is subtracted first: every shifted
    unnormalised probability is at most 1 in every mode ([FA-backward] §3.1, §3.2)."""
    rng = np.random.default_rng(12)
    q, k, v = rng.standard_normal((64, 16)) * 2.0, rng.standard_normal((64, 16)) * 2.0, rng.standard_normal((64, 16))
    scale = 0.6
    s = scale * q @ k.T
    assert s.max() > 12.0
    assert np.isinf(oracle.fp16_round(np.exp(s))).any()
    for mode in (0, 1, 2):
        fr = oracle.forward(q, k, v, False, scale, BETA, mode, elem="f16")
        p_hat = np.exp(s - fr.m[:, None])
        assert p_hat.max() <= 1.0 + 1e-12 and np.all(np.isfinite(oracle.fp16_round(p_hat)))
        assert np.all(np.isfinite(fr.o)) and np.all(np.isfinite(fr.lse))


def test_pages_printed_numbers():
    g = json.load(open(os.path.join(GOLDEN, "pages_numbers.json")))
    assert np.float16(g["fp16_max"]["value"]) == np.finfo(np.float16).max
    assert abs(float(np.finfo(np.float16).smallest_subnormal) - g["fp16_min_positive"]["value"]) < 1e-9
    for key in ("exp_11", "exp_12"):
        x = 11.0 if key == "exp_11" else 12.0
        assert abs(math.exp(x) - g[key]["value"]) < 1.0  # the page prints the value truncated
        assert np.isfinite(np.float16(math.exp(x))) == g[key]["fits_fp16"]
    # bf16: 8 exponent bits, 7 stored mantissa bits => spacing just above 1 is 2^-7
    assert g["bf16_mantissa_bits"]["value"] == 7
    assert oracle.bf16_round(1 + 2 ** -8 + 2 ** -10) == 1 + 2 ** -7
    assert float(torch.finfo(torch.bfloat16).max) > 3e38  # fp32's exponent range (8 bits)
    assert g["beta_range"]["value"][0] <= g["beta_default"]["value"] <= g["beta_range"]["value"][1]


# ----------------------------------------------------------------------------------------------
# P1: brute force, scalar Python loops, no shift at all


def _brute_force(q, k, v, causal, scale):
    n, d = len(q), len(q[0])
    o = [[0.0] * len(v[0]) for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        keys = [j for j in range(len(k)) if (not causal or j <= i)]
        e = {}
        for j in keys:
            s = 0.0
            for c in range(d):
                s += q[i][c] * k[j][c]
            e[j] = math.exp(scale * s)
        z = sum(e.values())
        lse[i] = math.log(z)
        for c in range(len(v[0])):
            o[i][c] = sum(e[j] * v[j][c] for j in keys) / z
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_brute_force_tiny(causal, mode):
    rng = np.random.default_rng(11 + mode)
    for n, d in [(1, 3), (5, 4), (16, 8)]:
        q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
        if n > 3:
            k[3] = k[1]  # a repeated key
            q[2] = k[1]
        o_ref, lse_ref = _brute_force(q.tolist(), k.tolist(), v.tolist(), causal, 0.7)
        fr = oracle.forward(q, k, v, causal, 0.7, BETA, mode)
        np.testing.assert_allclose(fr.o, o_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(fr.lse, lse_ref, rtol=1e-12, atol=1e-12)
        # row range of the scaled scores, by scalar loops over the visible keys
        for i in range(n):
            vis = [0.7 * sum(a * b for a, b in zip(q[i], k[j])) for j in range(n) if not causal or j <= i]
            assert math.isclose(fr.rm[i], max(vis), rel_tol=1e-12, abs_tol=1e-12)
            assert math.isclose(fr.smin[i], min(vis), rel_tol=1e-12, abs_tol=1e-12)


# ----------------------------------------------------------------------------------------------
# P2, P3: normalisation and shift invariance


@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    t = _head(make_inputs(3, B=1, H=1, N=256))
    fr = oracle.forward(t["q"], t["k"], t["v"], causal, 0.125)
    rows = np.arange(256)
    p = oracle.probabilities(t["q"], t["k"], 0.125, fr.lse, oracle.visible(rows, 256, causal))
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p[~oracle.visible(rows, 256, causal)] == 0)


@pytest.mark.parametrize("kind", ["grid", "sink", "dup"])
def test_shift_cancels_between_modes(kind):
    cid = {"grid": 5, "sink": 3, "dup": 1}[kind]
    t = _head(make_inputs(cid, B=1, H=1, N=128, d=64))
    outs = [oracle.forward(t["q"], t["k"], t["v"], True, 0.125, BETA, mode) for mode in (0, 1, 2)]
    for fr in outs[1:]:
        np.testing.assert_allclose(fr.o, outs[0].o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(fr.lse, outs[0].lse, rtol=1e-12, atol=1e-12)
    # the shift is really different where it should be
    assert np.any(outs[2].m != outs[0].m)


# ----------------------------------------------------------------------------------------------
# P4: tiled recurrence == untiled definition


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("bc", [1, 7, 32, 64, 200])
def test_tiled_recurrence_matches_untiled(causal, mode, bc):
    t = _head(grid_inputs(1, 1, 200, 16, seed=5))
    fr = oracle.forward(t["q"], t["k"], t["v"], causal, 0.3, BETA, mode)
    tr = oracle.tiled_forward(t["q"], t["k"], t["v"], causal, 0.3, BETA, mode, bc=bc)
    np.testing.assert_allclose(tr["o"], fr.o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(tr["lse"], fr.lse, rtol=1e-12, atol=1e-12)
    assert np.array_equal(tr["c"], fr.rs)
    assert np.array_equal(tr["r"], fr.rm)


def test_tiled_order_does_not_change_result():
    t = _head(make_inputs(3, B=1, H=1, N=192))
    a = oracle.tiled_forward(t["q"], t["k"], t["v"], False, 0.125, BETA, 1, bc=64)
    b = oracle.tiled_forward(t["q"], t["k"], t["v"], False, 0.125, BETA, 1, bc=64, order=[2, 0, 1])
    np.testing.assert_allclose(a["o"], b["o"], rtol=1e-12, atol=1e-12)
    assert np.array_equal(a["c"], b["c"])


# ----------------------------------------------------------------------------------------------
# P5: finite differences of L = sum(dO * O)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ties", [False, True])
def test_gradients_match_finite_differences(causal, ties):
    rng = np.random.default_rng(3 + 2 * causal + ties)
    n, d, scale = 8, 8, 0.5
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    if ties:
        k[5] = k[2]
        q[6] = k[2]
    br = oracle.backward(q, k, v, do, causal, scale)

    def loss(qq, kk, vv):
        return float(np.sum(do * oracle.forward(qq, kk, vv, causal, scale).o))

    h = 1e-6
    for name, grad in (("q", br.dq), ("k", br.dk), ("v", br.dv)):
        fd = np.zeros((n, d))
        for i in range(n):
            for c in range(d):
                args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
                args[name][i, c] += h
                lp = loss(args["q"], args["k"], args["v"])
                args[name][i, c] -= 2 * h
                lm = loss(args["q"], args["k"], args["v"])
                fd[i, c] = (lp - lm) / (2 * h)
        scale_ref = max(1.0, np.abs(grad).max())
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-6 * scale_ref, err_msg=name)


# ----------------------------------------------------------------------------------------------
# P6: closed forms


def test_closed_forms_causal_row0_constant_v_zero_q():
    rng = np.random.default_rng(21)
    n, d, scale = 64, 16, 0.25
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    fr = oracle.forward(q, k, v, True, scale)
    np.testing.assert_allclose(fr.o[0], v[0], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(fr.lse[0], scale * q[0] @ k[0], rtol=1e-14, atol=1e-14)
    br = oracle.backward(q, k, v, do, True, scale)
    np.testing.assert_allclose(br.dq[0], 0.0, atol=1e-14)

    vc = np.tile(rng.standard_normal(d), (n, 1))
    for causal in (False, True):
        fr = oracle.forward(q, k, vc, causal, scale)
        np.testing.assert_allclose(fr.o, vc, rtol=1e-13, atol=1e-13)

    q0 = np.zeros((n, d))
    for causal in (False, True):
        fr = oracle.forward(q0, k, v, causal, scale)
        cnt = np.arange(1, n + 1) if causal else np.full(n, n)
        mean = np.cumsum(v, axis=0) / cnt[:, None] if causal else np.tile(v.mean(axis=0), (n, 1))
        np.testing.assert_allclose(fr.o, mean, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(fr.lse, np.log(cnt), rtol=1e-14, atol=1e-14)


# ----------------------------------------------------------------------------------------------
# P7: the tie closed form of the BF16 article §3.2 (k equal maxima)


@pytest.mark.parametrize("n_ties", [2, 3, 5])
@pytest.mark.parametrize("s_max", [2.0, 0.75, -1.5])
def test_tie_closed_form(n_ties, s_max):
    others = [s_max - 9.0, s_max - 11.5, s_max - 30.0]
    values = [s_max] * n_ties + others
    q, k = _scores_row(values)
    v = np.eye(len(values))  # O = P, so the output row is the probability row
    tail = sum(math.exp(x - s_max) for x in others)
    for mode in (0, 1, 2):
        fr = oracle.forward(q, k, v, False, 1.0, BETA, mode)
        # normalised probability at each tied maximum: 1 / (k + tail), in every mode
        np.testing.assert_allclose(fr.o[0, :n_ties], 1.0 / (n_ties + tail), rtol=1e-13)
        assert fr.rs[0] == n_ties
        p_hat_max = math.exp(s_max - fr.m[0])
        if mode == 0:
            assert fr.m[0] == s_max and p_hat_max == 1.0 and fr.ones[0] == n_ties
        elif s_max > 0:
            # stabilised: P^ at the max = exp(-(beta - 1) * s_max) < 1
            assert fr.m[0] == BETA * s_max
            assert abs(p_hat_max - math.exp(-(BETA - 1) * s_max)) < 1e-15
            assert fr.ones[0] == 0
        else:
            # negative maximum: m = 0, P^ = exp(s_max)
            assert fr.m[0] == 0.0
            assert abs(p_hat_max - math.exp(s_max)) < 1e-15
            assert fr.ones[0] == 0


def test_shift_rule_without_repeats():
    q, k = _scores_row([2.0, 1.0, -3.0])
    v = np.eye(3)
    assert oracle.forward(q, k, v, False, 1.0, BETA, 1).m[0] == 2.0  # unique max: no shift
    assert oracle.forward(q, k, v, False, 1.0, BETA, 2).m[0] == 2.5  # anticipating rule shifts
    q, k = _scores_row([0.0, 0.0, -3.0])  # rm == 0 with a repeat: no branch fires
    fr = oracle.forward(q, k, np.eye(3), False, 1.0, BETA, 1)
    assert fr.m[0] == 0.0 and fr.ones[0] == 2


# ----------------------------------------------------------------------------------------------
# P8: repeat counts by exact integer arithmetic on grid inputs


def test_dupcount_by_integer_arithmetic():
    t = grid_inputs(1, 2, 384, 64, seed=99)
    for h in range(2):
        q = t["q"][0, h].to(torch.float64).numpy()
        k = t["k"][0, h].to(torch.float64).numpy()
        qi = np.rint(2 * q).astype(np.int64)  # grid entries are multiples of 0.5
        ki = np.rint(2 * k).astype(np.int64)
        x4 = qi @ ki.T  # 4 * (q . k), exact
        for causal in (False, True):
            mask = oracle.visible(np.arange(384), 384, causal)
            xm = np.where(mask, x4, np.iinfo(np.int64).min)
            mx = xm.max(axis=1)
            rs = np.sum(xm == mx[:, None], axis=1)
            fr = oracle.forward(q, k, q, causal, 0.0883883461356163, BETA, 1)
            assert np.array_equal(fr.rs, rs)
            assert rs.max() > 1  # the grid really produces ties


@pytest.mark.parametrize("causal", [0, 1, 2])
@pytest.mark.parametrize("nq,nk", [(333, 333), (96, 416), (416, 96)])
def test_integer_repeat_counts_match_the_scaled_scores(causal, nq, nk):
    t = rect_inputs(1, 1, nq, nk, 64, seed=nq + 7 * nk + causal, grid=True)
    q, k = _np(t["q"][0, 0]), _np(t["k"][0, 0])
    xmax, cnt = oracle.integer_repeat_counts(2 * q, 2 * k, causal, row_chunk=100)
    s = oracle.scaled_scores(q, k, 0.0883883461356163, oracle.visible(np.arange(nq), nk, causal, nq))
    rm, rs = oracle.row_max_and_repeats(s)
    assert np.array_equal(cnt, rs)
    live = rs > 0
    assert np.array_equal(xmax[live] * 0.25 * 0.0883883461356163, rm[live])
    assert rs.max() > 1


def test_integer_repeat_counts_brute_force_and_guards():
    rng = np.random.default_rng(5)
    qi = rng.integers(-2, 3, (9, 5)).astype(np.float64)
    ki = rng.integers(-2, 3, (11, 5)).astype(np.float64)
    for causal in (0, 1, 2):
        xmax, cnt = oracle.integer_repeat_counts(qi, ki, causal, row_chunk=4)
        off = {0: None, 1: 0, 2: 11 - 9}[causal]
        for i in range(9):
            vals = [int(sum(qi[i, t] * ki[j, t] for t in range(5))) for j in range(11)
                    if off is None or j <= i + off]
            if not vals:
                assert cnt[i] == 0
                continue
            assert xmax[i] == max(vals) and cnt[i] == vals.count(max(vals))
    with pytest.raises(ValueError):
        oracle.integer_repeat_counts(qi + 0.5, ki, 0)
    with pytest.raises(ValueError):
        oracle.integer_repeat_counts(qi * 4096, ki * 4096, 0)


def test_tied_maxima_construction():
    """The constructed rows attain their maximum exactly at the two tie keys, with the sign asked
    for; the rule then gives beta rm, 0 and 0 (closed form of [BF16-FA] §4.1)."""
    for d in (64, 128):
        t, rows = tied_maxima_inputs(300, d, seed=3 + d)
        x = _head(t)
        scale = 0.125 if d == 64 else 0.0883883461356163
        fr = oracle.forward(x["q"], x["k"], x["v"], False, scale, 1.5, 1)
        s = scale * x["q"] @ x["k"].T
        for kind, rr in rows.items():
            if kind == "allzero":
                assert np.all(s[rr] == 0.0) and np.all(fr.rs[rr] == 300)
                continue
            assert np.all(np.argsort(-s[rr], axis=1, kind="stable")[:, :2] == [7, 200])
            assert np.all(fr.rs[rr] == 2)
            sign = {"pos": 1, "neg": -1, "zero": 0}[kind]
            assert np.all(np.sign(fr.rm[rr]) == sign)
            assert np.all(fr.m[rr] == (1.5 * fr.rm[rr] if kind == "pos" else 0.0))


def test_dupcount_config1_construction():
    t = _head(make_inputs(1))
    fr = oracle.forward(t["q"], t["k"], t["v"], False, 0.125, BETA, 0)
    assert np.all(fr.rs[:8] == 2)
    # any other row whose maximum falls on key 3 (= key 17) repeats too; all the rest are unique
    s = 0.125 * t["q"] @ t["k"].T
    on_dup = np.isin(np.argmax(s, axis=1), [3, 17])
    assert np.array_equal(fr.rs, np.where(on_dup, 2, 1))
    top2 = np.sort(0.125 * t["q"][:8] @ t["k"].T, axis=1)[:, -3:]
    assert np.all(top2[:, -1] == top2[:, -2])
    assert np.all(top2[:, -2] - top2[:, -3] > 1.0)


# ----------------------------------------------------------------------------------------------
# P9: gradient invariants


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    t = _head(make_inputs(2, B=1, H=1, N=256))
    scale = 0.125
    fr = oracle.forward(t["q"], t["k"], t["v"], causal, scale)
    br = oracle.backward(t["q"], t["k"], t["v"], t["do"], causal, scale)
    rows = np.arange(256)
    mask = oracle.visible(rows, 256, causal)
    p = oracle.probabilities(t["q"], t["k"], scale, fr.lse, mask)
    dp = t["do"] @ t["v"].T
    np.testing.assert_allclose(br.delta, np.sum(p * dp, axis=1), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(br.dk.sum(axis=0), 0.0, atol=1e-10)
    np.testing.assert_allclose(br.dv.sum(axis=0), t["do"].sum(axis=0), rtol=1e-11, atol=1e-10)
    np.testing.assert_allclose(np.sum(t["q"] * br.dq), np.sum(t["k"] * br.dk), rtol=1e-10, atol=1e-10)


# ----------------------------------------------------------------------------------------------
# P11: tile replay of the exact-1.0 count vs a scalar per-tile replay


# The interval of real values each 16-bit type rounds (RNE) to exactly 1.0, from the formats:
# bf16 spacing is 2^-8 below 1 and 2^-7 above, fp16 2^-11 below and 2^-10 above.  Both midpoints
# are ties, and 1.0 is the neighbour with the even last mantissa bit, so both round to 1.0.
ONE_WINDOW = {"bf16": (1 - 2 ** -9, 1 + 2 ** -8), "f16": (1 - 2 ** -12, 1 + 2 ** -11)}


def _scalar_tile_ones(q, k, causal, scale, beta, mode, bc, elem="bf16"):
    n = len(q)
    out = []
    for i in range(n):
        r, c, ones = -math.inf, 0, 0
        for j0 in range(0, len(k), bc):
            keys = [j for j in range(j0, min(len(k), j0 + bc)) if (not causal or j <= i)]
            if not keys:
                continue
            s = {j: scale * float(np.dot(q[i], k[j])) for j in keys}
            tm = max(s.values())
            tc = sum(1 for x in s.values() if x == tm)
            rn = max(r, tm)
            c = (tc if tm == rn else 0) + (c if r == rn else 0)
            r = rn
            rep = c > 1 if mode == 1 else (mode == 2)
            m = beta * r if (r > 0 and rep) else (0.0 if (r < 0 and rep) else r)
            lo, hi = ONE_WINDOW[elem]
            for x in s.values():
                if lo <= math.exp(x - m) <= hi:
                    ones += 1
        out.append(ones)
    return np.array(out)


@pytest.mark.parametrize("elem", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_tile_ones_vs_scalar_replay(causal, mode, elem):
    t = _head(grid_inputs(1, 1, 48, 8, seed=17))
    scale = 0.35
    want = _scalar_tile_ones(t["q"], t["k"], causal, scale, BETA, mode, 16, elem)
    got = oracle.tiled_ones(t["q"], t["k"], causal, scale, BETA, mode, bc=16, elem=elem)
    got2 = oracle.tiled_forward(t["q"], t["k"], t["v"], causal, scale, BETA, mode, bc=16, elem=elem)["ones"]
    assert np.array_equal(got, want)
    assert np.array_equal(got2, want)


def test_mode1_residual_and_mode2_zero():
    # max 2.0 at key 1 (block 0) repeated at key 5 (block 1) with bc = 4: mode 1 emits one exact
    # 1.0 (at key 1, before the repeat is seen); mode 2 and the untiled rule emit none.
    q, k = _scores_row([0.5, 2.0, -1.0, 0.25, 1.0, 2.0, -2.0, 0.0])
    v = np.eye(8)
    assert oracle.tiled_forward(q, k, v, False, 1.0, BETA, 1, bc=4)["ones"][0] == 1
    assert oracle.tiled_forward(q, k, v, False, 1.0, BETA, 2, bc=4)["ones"][0] == 0
    assert oracle.forward(q, k, v, False, 1.0, BETA, 1).ones[0] == 0
    assert oracle.tiled_forward(q, k, v, False, 1.0, BETA, 1, bc=8)["ones"][0] == 0


def test_mode2_no_ones_on_grid_away_from_zero():
    t = _head(grid_inputs(1, 1, 512, 128, seed=5))
    scale = 0.0883883461356163
    fr = oracle.forward(t["q"], t["k"], t["v"], True, scale, BETA, 0)
    ones = oracle.tiled_ones(t["q"], t["k"], True, scale, BETA, 2, bc=64)
    away = fr.rm != 0
    assert np.all(ones[away] == 0)
    ones1 = oracle.tiled_ones(t["q"], t["k"], True, scale, BETA, 1, bc=64)
    assert ones1[away].sum() > 0  # the tie-conditional rule leaves some, as predicted


# ----------------------------------------------------------------------------------------------
# Planted mistakes: the pins above must reject a plausibly wrong oracle.  Each mutation is built
# here, on the CPU, from the oracle's own pieces with one term changed.


def _fd_gradient_error(backward_fn, causal=True):
    rng = np.random.default_rng(5)
    n, d, scale = 8, 8, 0.5
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    grads = backward_fn(q, k, v, do, causal, scale)
    worst = 0.0
    h = 1e-6
    for idx, (name, base) in enumerate((("q", q), ("k", k), ("v", v))):
        for i in range(n):
            for c in range(d):
                args = [q.copy(), k.copy(), v.copy()]
                args[idx][i, c] += h
                lp = np.sum(do * oracle.forward(*args, causal, scale).o)
                args[idx][i, c] -= 2 * h
                lm = np.sum(do * oracle.forward(*args, causal, scale).o)
                worst = max(worst, abs(grads[idx][i, c] - (lp - lm) / (2 * h)))
    return worst


def _backward_variant(q, k, v, do, causal, scale, flaw):
    fr = oracle.forward(q, k, v, causal, scale)
    n = len(q)
    mask = oracle.visible(np.arange(n), n, causal)
    p = oracle.probabilities(q, k, scale, fr.lse, mask)
    delta = np.sum(do * fr.o, axis=1)
    if flaw == "delta_sign":
        delta = -delta
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - delta[:, None])
    if flaw == "drop_delta":
        ds = p * dp
    dq = scale * ds @ k
    dk = scale * ds.T @ q
    if flaw == "transposed_dk":
        dk = scale * ds @ q
    if flaw == "missing_scale":
        dq = ds @ k
    return dq, dk, dv


def test_planted_gradient_mistakes_are_caught():
    good = _fd_gradient_error(lambda *a: _backward_variant(*a, flaw=None))
    assert good < 1e-6
    for flaw in ("delta_sign", "drop_delta", "transposed_dk", "missing_scale"):
        assert _fd_gradient_error(lambda *a: _backward_variant(*a, flaw=flaw)) > 1e-3, flaw


def test_planted_shift_mistakes_are_caught():
    # a shift that forgets beta, or shifts negative maxima by beta, breaks the tie closed form
    rm = np.array([2.0, -1.5])
    rs = np.array([3, 3])
    good = oracle.stable_shift(rm, rs, BETA, 1)
    assert good[0] == BETA * 2.0 and good[1] == 0.0
    forgot_beta = np.where((rm > 0) & (rs > 1), 1.0 * rm, rm)
    assert math.exp(2.0 - forgot_beta[0]) == 1.0  # the exact 1.0 the rule exists to avoid
    wrong_neg = np.where(rs > 1, BETA * rm, rm)
    assert math.exp(-1.5 - wrong_neg[1]) > 1.0  # P^ above 1 for a negative maximum


def test_planted_count_merge_mistake_is_caught():
    # merging tile counts without checking which maximum survives over-counts repeats
    t = _head(grid_inputs(1, 1, 128, 16, seed=3))
    good = oracle.tiled_forward(t["q"], t["k"], t["v"], False, 0.3, BETA, 1, bc=16)["c"]
    s = 0.3 * t["q"] @ t["k"].T
    r = np.full(128, -np.inf)
    c = np.zeros(128, dtype=np.int64)
    for j0 in range(0, 128, 16):
        blk = s[:, j0:j0 + 16]
        tm = blk.max(axis=1)
        tc = np.sum(blk == tm[:, None], axis=1)
        c = c + tc  # the planted mistake: counts of smaller maxima leak in
        r = np.maximum(r, tm)
    assert np.array_equal(good, oracle.forward(t["q"], t["k"], t["v"], False, 0.3, BETA, 1).rs)
    assert not np.array_equal(c, good)


def test_row_subset_functions_match_full_oracle():
    """forward_rows and dq_rows (used to check sampled rows at sequence lengths the full oracle
    cannot afford) evaluate the same definitions as forward/backward on any subset of rows, in
    any order, with the causal mask taken from the absolute row index."""
    rng = np.random.default_rng(5)
    n, d = 70, 16
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    rows = np.array([69, 0, 33, 1, 64, 17])
    for causal in (False, True):
        for mode in (0, 1, 2):
            full = oracle.forward(q, k, v, causal, 0.3, 1.25, mode, row_chunk=16)
            part = oracle.forward_rows(q, k, v, rows, causal, 0.3, 1.25, mode)
            for name in ("o", "lse", "rm", "rs", "m", "l", "ones", "smin"):
                assert np.array_equal(getattr(part, name), getattr(full, name)[rows]), name
        br = oracle.backward(q, k, v, do, causal, 0.3, row_chunk=16)
        dq, delta = oracle.dq_rows(q, k, v, do, rows, causal, 0.3)
        np.testing.assert_allclose(dq, br.dq[rows], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(delta, br.delta[rows], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------------------------
# P11: Nq != Nk and the two causal alignments.  Top-left: query i sees keys j <= i.  Bottom-right:
# the last query sees every key and each earlier query one key fewer, i.e. the query's distance
# from the last query is at most the key's distance from the last key.  A query that sees no key
# has the empty softmax sum: O = 0, LSE = -inf, zero gradients.


def _sees(i, j, nq, nk, causal):
    if causal == 0:
        return True
    if causal == 1:
        return j <= i
    return (nq - 1 - i) <= (nk - 1 - j)


def _brute_force_rect(q, k, v, do, causal, scale):
    """Scalar loops: O, LSE and, by the chain rule written per element, dQ, dK, dV."""
    nq, nk, d, dv_ = len(q), len(k), len(q[0]), len(v[0])
    o = [[0.0] * dv_ for _ in range(nq)]
    lse = [-math.inf] * nq
    dq = [[0.0] * d for _ in range(nq)]
    dk = [[0.0] * d for _ in range(nk)]
    dv = [[0.0] * dv_ for _ in range(nk)]
    for i in range(nq):
        keys = [j for j in range(nk) if _sees(i, j, nq, nk, causal)]
        if not keys:
            continue
        e = {j: math.exp(scale * sum(q[i][c] * k[j][c] for c in range(d))) for j in keys}
        z = sum(e.values())
        lse[i] = math.log(z)
        p = {j: e[j] / z for j in keys}
        for c in range(dv_):
            o[i][c] = sum(p[j] * v[j][c] for j in keys)
        # dL/dp_j = do_i . v_j; softmax Jacobian: dS_j = p_j (dL/dp_j - sum_l p_l dL/dp_l)
        g = {j: sum(do[i][c] * v[j][c] for c in range(dv_)) for j in keys}
        gbar = sum(p[j] * g[j] for j in keys)
        for j in keys:
            ds = p[j] * (g[j] - gbar)
            for c in range(d):
                dq[i][c] += scale * ds * k[j][c]
                dk[j][c] += scale * ds * q[i][c]
            for c in range(dv_):
                dv[j][c] += p[j] * do[i][c]
    return tuple(np.array(x) for x in (o, lse, dq, dk, dv))


@pytest.mark.parametrize("causal", [0, 1, 2])
@pytest.mark.parametrize("nq,nk", [(3, 7), (7, 3), (1, 5), (5, 1), (6, 6), (9, 4)])
def test_brute_force_rectangular(causal, nq, nk):
    rng = np.random.default_rng(100 * nq + nk + causal)
    d = 4
    q, do = rng.standard_normal((nq, d)), rng.standard_normal((nq, d))
    k, v = rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    o, lse, dq, dk, dv = _brute_force_rect(q.tolist(), k.tolist(), v.tolist(), do.tolist(), causal, 0.6)
    for mode in (0, 1, 2):
        fr = oracle.forward(q, k, v, causal, 0.6, BETA, mode)
        np.testing.assert_allclose(fr.o, o, rtol=1e-12, atol=1e-12)
        assert np.array_equal(np.isinf(fr.lse), np.isinf(lse))
        fin = np.isfinite(lse)
        np.testing.assert_allclose(fr.lse[fin], lse[fin], rtol=1e-12, atol=1e-12)
        assert np.all(fr.lse[~fin] == -np.inf)
        tr = oracle.tiled_forward(q, k, v, causal, 0.6, BETA, mode, bc=2)
        np.testing.assert_allclose(tr["o"], o, rtol=1e-12, atol=1e-12)
        assert np.array_equal(tr["lse"][~fin], lse[~fin])
    br = oracle.backward(q, k, v, do, causal, 0.6)
    np.testing.assert_allclose(br.dq, dq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(br.dk, dk, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(br.dv, dv, rtol=1e-10, atol=1e-12)
    vis = oracle.visible(np.arange(nq), nk, causal, nq)
    assert int(vis.sum()) == oracle.visible_pairs(nq, nk, causal)
    for i in range(nq):
        for j in range(nk):
            assert vis[i, j] == _sees(i, j, nq, nk, causal)


def test_bottom_right_is_the_tail_of_a_square_problem():
    """Bottom-right with Nq < Nk: the queries sit at the last Nq positions of an Nk x Nk causal
    problem.  O, LSE and the counts equal that problem's last rows; dK and dV equal its
    gradients when the first Nk - Nq rows carry no output gradient."""
    rng = np.random.default_rng(8)
    nk, nq, d = 45, 13, 8
    qf, kf, vf, dof = (rng.standard_normal((nk, d)) for _ in range(4))
    kf[30] = kf[7]
    qf[40] = kf[7]
    dof[: nk - nq] = 0.0
    for mode in (0, 1, 2):
        sq = oracle.forward(qf, kf, vf, True, 0.4, BETA, mode)
        br = oracle.forward(qf[nk - nq:], kf, vf, 2, 0.4, BETA, mode)
        for name in ("o", "lse", "rm", "rs", "m", "l", "ones", "smin"):
            np.testing.assert_array_equal(getattr(br, name), getattr(sq, name)[nk - nq:], err_msg=name)
    gs = oracle.backward(qf, kf, vf, dof, True, 0.4)
    gb = oracle.backward(qf[nk - nq:], kf, vf, dof[nk - nq:], 2, 0.4)
    np.testing.assert_allclose(gb.dq, gs.dq[nk - nq:], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gb.dk, gs.dk, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gb.dv, gs.dv, rtol=1e-12, atol=1e-13)
    # and it differs from top-left on the same rectangular problem
    tl = oracle.forward(qf[nk - nq:], kf, vf, 1, 0.4)
    assert not np.allclose(tl.o, oracle.forward(qf[nk - nq:], kf, vf, 2, 0.4).o)


def test_more_queries_than_keys():
    """Nq > Nk.  Top-left: rows from Nk - 1 on see every key (the non-causal result).
    Bottom-right: the first Nq - Nk rows see nothing (O = 0, LSE = -inf, no gradient); the rest
    are the Nk x Nk causal problem of those rows."""
    rng = np.random.default_rng(9)
    nq, nk, d = 21, 8, 8
    q, do = rng.standard_normal((nq, d)), rng.standard_normal((nq, d))
    k, v = rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    tl = oracle.forward(q, k, v, 1, 0.5)
    full = oracle.forward(q, k, v, 0, 0.5)
    np.testing.assert_array_equal(tl.o[nk - 1:], full.o[nk - 1:])
    np.testing.assert_array_equal(tl.lse[nk - 1:], full.lse[nk - 1:])
    e = nq - nk
    brf = oracle.forward(q, k, v, 2, 0.5, BETA, 2)
    assert np.all(brf.o[:e] == 0) and np.all(brf.lse[:e] == -np.inf) and np.all(brf.l[:e] == 0)
    assert np.all(brf.rs[:e] == 0) and np.all(brf.ones[:e] == 0) and np.all(brf.smin[:e] == np.inf)
    assert np.all(brf.rm[:e] == -np.inf)
    sq = oracle.forward(q[e:], k, v, 1, 0.5, BETA, 2)
    np.testing.assert_array_equal(brf.o[e:], sq.o)
    np.testing.assert_array_equal(brf.lse[e:], sq.lse)
    gb = oracle.backward(q, k, v, do, 2, 0.5)
    gs = oracle.backward(q[e:], k, v, do[e:], 1, 0.5)
    assert np.all(gb.dq[:e] == 0) and np.all(gb.delta[:e] == 0)
    np.testing.assert_allclose(gb.dq[e:], gs.dq, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gb.dk, gs.dk, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gb.dv, gs.dv, rtol=1e-12, atol=1e-13)


def test_no_keys_and_single_query():
    rng = np.random.default_rng(10)
    q, do = rng.standard_normal((5, 4)), rng.standard_normal((5, 4))
    k = v = np.zeros((0, 4))
    for causal in (0, 1, 2):
        fr = oracle.forward(q, k, v, causal, 0.5, BETA, 1)
        assert np.all(fr.o == 0) and np.all(fr.lse == -np.inf)
        br = oracle.backward(q, k, v, do, causal, 0.5)
        assert br.dq.shape == (5, 4) and np.all(br.dq == 0) and br.dk.shape == (0, 4)
    # one query, bottom-right: it sees every key, so the result is the non-causal one
    k, v = rng.standard_normal((9, 4)), rng.standard_normal((9, 4))
    a = oracle.forward(q[:1], k, v, 2, 0.5)
    b = oracle.forward(q[:1], k, v, 0, 0.5)
    np.testing.assert_array_equal(a.o, b.o)
    assert oracle.visible_pairs(1, 9, 1) == 1 and oracle.visible_pairs(1, 9, 2) == 9


def test_visible_pairs_closed_forms():
    for nq, nk in [(8192, 8192), (100, 300), (300, 100), (1, 1), (0, 5), (5, 0)]:
        assert oracle.visible_pairs(nq, nk, 0) == nq * nk
        if nq <= nk:
            assert oracle.visible_pairs(nq, nk, 1) == nq * (nq + 1) // 2
            assert oracle.visible_pairs(nq, nk, 2) == nq * nk - nq * (nq - 1) // 2
        else:
            assert oracle.visible_pairs(nq, nk, 1) == nk * (nk + 1) // 2 + (nq - nk) * nk
            assert oracle.visible_pairs(nq, nk, 2) == nk * (nk + 1) // 2
    assert oracle.visible_pairs(8192, 8192, 1) == oracle.exact_causal_pairs(8192)


# ---- FP8 P^ V variant ---------------------------------------------------------------------------


def _torch_e4m3(x):
    """Round through torch's float8_e4m3fn cast (an independent implementation of the format)."""
    import torch
    t = torch.tensor(np.asarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_round_matches_torch_cast_and_closed_forms():
    rng = np.random.default_rng(8)
    mags = np.exp2(rng.uniform(-12.0, np.log2(440.0), 200000))
    x = (mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32).astype(np.float64)
    # exact midpoints between neighbours, in every normal binade up to 256 and in the subnormals
    ties = [(np.arange(0, 8) + 0.5) * 2.0**-9]
    ties += [(np.arange(8, 16) + 0.5) * 2.0**(e - 3) for e in range(-6, 8)]
    x = np.concatenate([x, *ties, -np.concatenate(ties), [0.0, 448.0, -448.0, 2.0**-9, 2.0**-6]])
    assert np.array_equal(oracle.e4m3_round(x), _torch_e4m3(x))
    # closed forms: 4 significant bits, ties to even, 2^-9 subnormal spacing, 448 the largest value
    assert oracle.e4m3_round(1.0625) == 1.0 and oracle.e4m3_round(1.1875) == 1.25
    assert oracle.e4m3_round(2.0**-10) == 0.0 and oracle.e4m3_round(3 * 2.0**-10) == 2.0**-8
    assert oracle.e4m3_round(448.0) == 448.0 and np.isnan(oracle.e4m3_round(500.0))
    assert oracle.e4m3_round(252.0) == 256.0 and oracle.e4m3_round(247.0) == 240.0


def test_fp8_p_hat_rounding_and_exact_one():
    # P^ is fed as e4m3(256 P^) / 256: the spacing just below 1 is 1/16, so P^ >= 0.96875 gives 1.0
    assert oracle.fp8_p_hat_round(1.0) == 1.0 and oracle.fp8_p_hat_round(0.97) == 1.0
    assert oracle.fp8_p_hat_round(0.968) == 0.9375
    # small probabilities keep 4 significant bits down to 2^-14, then the 2^-17 subnormal spacing
    assert oracle.fp8_p_hat_round(2.0**-14 * 1.0625) == 2.0**-14
    assert oracle.fp8_p_hat_round(2.0**-18) == 0.0 and oracle.fp8_p_hat_round(3 * 2.0**-18) == 2.0**-16


def _brute_fp8_forward(q, k, v, causal, scale):
    """Scalar loops, mode 0, one key block: the FP8 P^ V definition written out, with torch's cast
    as the rounding routine."""
    n, nk = q.shape[0], k.shape[0]
    amax = np.float32(max(abs(float(x)) for x in v.ravel()))
    s = amax / np.float32(448.0) if amax > 0 else np.float32(1.0)
    inv = np.float32(1.0) / s
    vq = np.array([[float(_torch_e4m3(np.float32(float(v[j, c])) * inv)) * float(s) for c in range(v.shape[1])]
                   for j in range(nk)])
    o = np.zeros((n, v.shape[1]))
    for i in range(n):
        keys = [j for j in range(nk) if (not causal) or j <= i]
        sc = [scale * sum(float(q[i, t]) * float(k[j, t]) for t in range(q.shape[1])) for j in keys]
        m = max(sc)
        p = [math.exp(x - m) for x in sc]
        l = sum(p)
        for idx, j in enumerate(keys):
            pq = float(_torch_e4m3(np.float32(256.0 * p[idx]))) / 256.0
            o[i] += pq * vq[j] / l
    return o


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_pv_tiled_forward_brute_force(causal):
    rng = np.random.default_rng(81 + int(causal))
    n, d = 12, 8
    q = oracle.bf16_round(rng.standard_normal((n, d)))
    k = oracle.bf16_round(rng.standard_normal((n, d)))
    v = oracle.bf16_round(rng.standard_normal((n, d)))
    got = oracle.tiled_forward(q, k, v, causal, 0.35, mode=0, bc=128, pv="fp8")["o"]
    want = _brute_fp8_forward(q, k, v, causal, 0.35)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def _fp8_bound(x, fr, scale, n):
    mask = np.ones((n, n), dtype=bool)
    p = oracle.probabilities(x["q"], x["k"], scale, fr.lse, mask)
    return (p @ np.abs(x["v"])) * (2.0**-4 + 2.0**-4 + 2.0**-8) + 2.0**-14 * np.abs(x["v"]).max()


def test_fp8_pv_replay_keeps_rows_with_large_shifts(monkeypatch):
    """Rows whose repeated maximum is +-58 or +-116 (tied_maxima_inputs, d = 128): under the rule
    every P^ of the row is at most e^{-(beta-1) rm} or e^{rm}, so e4m3(2^8 P^) would be 0.  With the
    variant's range adjustment the replay stays within the E4M3 rounding bound of the exact O; a
    replay that drops the adjustment (planted) returns O = 0 there and fails the same bound."""
    t, rows = tied_maxima_inputs(300, 128, seed=2400)
    x = _head(t)
    scale = 0.0883883461356163
    big = [r for r in rows["pos"] + rows["neg"]]
    for mode in (1, 2):
        fr = oracle.forward(x["q"], x["k"], x["v"], False, scale, BETA, mode)
        big = [r for r in rows["pos"] + rows["neg"] if abs(fr.rm[r]) >= 40.0]
        assert len(big) == 8 and np.all(np.exp(fr.rm[big] - fr.m[big]) < 2.0**-18)  # 2^8 P^ < 2^-10
        f8 = oracle.tiled_forward(x["q"], x["k"], x["v"], False, scale, BETA, mode, bc=128, pv="fp8")
        bound = _fp8_bound(x, fr, scale, 300)
        err = np.abs(f8["o"] - fr.o)
        assert np.all(err[big] <= bound[big])
        assert np.abs(fr.o[big]).max() > 0.5
    import oracle.tiled as tiled
    plain = tiled.fp8_p_hat_round
    monkeypatch.setattr(tiled, "fp8_p_hat_round", lambda p, extra=0: plain(p))
    f8 = oracle.tiled_forward(x["q"], x["k"], x["v"], False, scale, BETA, 2, bc=128, pv="fp8")
    assert np.all(f8["o"][big] == 0.0)
    assert not np.all(np.abs(f8["o"] - fr.o)[big] <= _fp8_bound(x, fr, scale, 300)[big])


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_fp8_pv_forward_within_rounding_bound(mode):
    """Quantised against exact, per element: |O_q - O| <= sum_j P_j |v_j| (2^-4 + 2^-4 + 2^-8)
    + 2^-14 max|v| (relative rounding of P^ and of V, their product, and the subnormal floors of
    P^ and of V / s), with LSE unchanged."""
    rng = np.random.default_rng(90 + mode)
    n, d, bc = 300, 64, 128
    q = oracle.bf16_round(rng.standard_normal((n, d)))
    k = oracle.bf16_round(rng.standard_normal((n, d)))
    v = oracle.bf16_round(rng.standard_normal((n, d)) * np.linspace(0.1, 3.0, n)[:, None])
    for causal in (False, True):
        ex = oracle.tiled_forward(q, k, v, causal, d ** -0.5, mode=mode, bc=bc)
        f8 = oracle.tiled_forward(q, k, v, causal, d ** -0.5, mode=mode, bc=bc, pv="fp8")
        assert np.array_equal(ex["lse"], f8["lse"])
        fr = oracle.forward(q, k, v, causal, d ** -0.5)
        mask = oracle.visible(np.arange(n), n, causal, n)
        p = oracle.probabilities(q, k, d ** -0.5, fr.lse, mask)
        weight = p @ np.abs(v)
        bound = weight * (2.0**-4 + 2.0**-4 + 2.0**-8) + 2.0**-14 * np.abs(v).max()
        err = np.abs(f8["o"] - ex["o"])
        assert np.all(err <= bound), (err - bound).max()
        assert err.max() > 1e-4  # the rounding is really there
        assert np.allclose(ex["o"], fr.o, rtol=1e-12, atol=1e-12)

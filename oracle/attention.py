"""Plain fp64 CPU oracle for softmax attention with the stabilised row shift, forward and backward.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the CPU-baseline leg of
the benchmark may import this module.  The HIP library never calls it, and it shares no code
with the library.

Every quantity is computed in float64 with numpy, directly from its definition, on the exact
fp64 images of the bf16 inputs.  Rows are evaluated in chunks only to bound memory: softmax is a
per-row operation, and the gradient sums over rows are partial sums added in chunk order.

Pages the definitions follow (titles as they appear, sections as numbered there):
  [FA-practice]  "Flash Attention低精度训练稳定性优化实践" (jsqmd.com/news/761560)
  [BF16-FA]      the BF16 Flash Attention stability article at ijyty.com/news/896914
  [FA-backward]  "FlashAttention 训练时为什么会梯度爆炸？一次拆透反向传播的坑" (cnnetsun.cn/a/2497354)
  [WhyFail]      "為什么BF16的FlashAttention會把訓練「炸掉」？" (web578.cn/c/0305332L962026.html)

Readings where the pages are silent or garbled (the extraction of [BF16-FA] dropped the
comparison and assignment operators):
  * the conditional shift of [BF16-FA] §4.1 reads as strict comparisons: rm > 0 and rs > 1
    give m = beta * rm; rm < 0 and rs > 1 give m = 0; otherwise m = rm;
  * "mode 2" applies the same rule with the repeat count taken as at least 2, i.e. the shift
    is applied to every row whether or not a repeat has been seen yet;
  * causal masking is top-left aligned by default (key j visible to query i iff j <= i); the
    bottom-right alignment (j <= i + Nk - Nq) is the other option, and a row that sees no key
    has O = 0 and LSE = -inf (the log of an empty sum);
  * the saved logsumexp uses the natural log of the scaled scores: LSE = m + ln(l).
"""
from __future__ import annotations

import dataclasses

import numpy as np

MODE_STANDARD = 0
MODE_TIE_RULE = 1
MODE_TIE_ANTICIPATE = 2


def bf16_round(x):
    """Round float64 values to the nearest bfloat16 value, ties to even, returned as float64.

    bfloat16 keeps 8 significant bits (7 stored mantissa bits plus the implicit one) and the fp32
    exponent range [BF16-FA] §1.  Values are rounded directly from fp64 (no fp32 step).
    Subnormal and overflow handling is outside what this oracle needs: inputs here are
    probabilities in [0, 1] and bf16 tensors already.
    """
    x = np.asarray(x, dtype=np.float64)
    mant, expo = np.frexp(x)  # x = mant * 2**expo, |mant| in [0.5, 1)
    # 8 significant bits: scale the mantissa by 2**8 and round half to even (np.rint is RNE).
    return np.ldexp(np.rint(np.ldexp(mant, 8)), expo - 8)


CAUSAL_NONE = 0
CAUSAL_TOP_LEFT = 1
CAUSAL_BOTTOM_RIGHT = 2


def visible(rows, n_keys, causal, n_queries=None, keys=None):
    """Boolean [len(rows), n_keys] (or [len(rows), len(keys)] for a subset `keys` of the key
    indices): whether key j is visible to query row i.

    causal 0 / False: every key.  1 / True (top-left aligned): j <= i.  2 (bottom-right aligned,
    the last query sees every key): j <= i + n_keys - n_queries, so with more queries than keys
    the first n_queries - n_keys rows see no key at all.  n_queries is needed for 2 only; with
    n_queries == n_keys the two alignments coincide.
    """
    rows = np.asarray(rows)
    keys = np.arange(n_keys) if keys is None else np.asarray(keys)
    causal = int(causal)
    if causal == CAUSAL_NONE:
        return np.ones((rows.size, keys.size), dtype=bool)
    if causal == CAUSAL_TOP_LEFT:
        off = 0
    elif causal == CAUSAL_BOTTOM_RIGHT:
        if n_queries is None:
            raise ValueError("bottom-right alignment needs the number of queries")
        off = n_keys - n_queries
    else:
        raise ValueError(f"causal must be 0, 1 or 2, got {causal}")
    return keys[None, :] <= rows[:, None] + off


def fp16_round(x):
    """Round float64 values to the nearest IEEE binary16 value, ties to even, as float64.

    binary16 keeps 11 significant bits for normal values (|x| >= 2^-14) and a fixed spacing of
    2^-24 below that (subnormals, the 5.96e-8 lower end of the range [FA-practice] §2.1 gives);
    values that round above the largest finite value 65504 become +-inf ([FA-backward] §3.1:
    e^12 overflows, e^11 does not).  Rounded directly from fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    _, expo = np.frexp(x)  # x = mant * 2**expo, |mant| in [0.5, 1)
    e = np.maximum(expo, -13)  # below 2^-14 the spacing stays 2^-24 = 2^(-13 - 11)
    r = np.ldexp(np.rint(np.ldexp(x, 11 - e)), e - 11)
    return np.where(np.abs(r) > 65504.0, np.copysign(np.inf, x), r)


def e4m3_round(x):
    """Round float64 values to the nearest OCP FP8 E4M3 value (the "e4m3fn" encoding), ties to
    even, returned as float64.

    E4M3 keeps 4 significant bits (3 stored) for normal values (|x| >= 2^-6, exponent bias 7), a
    fixed spacing of 2^-9 below that (subnormals), and its largest finite value is 448 (the
    encoding has no infinity).  FP8 is the lower-precision format [BF16-FA] §6.1 extends the
    method to.  Magnitudes that round above 448 are outside what this oracle needs and come back
    as nan.  Rounded directly from fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    _, expo = np.frexp(x)  # x = mant * 2**expo, |mant| in [0.5, 1)
    e = np.maximum(expo, -5)  # below 2^-6 the spacing stays 2^-9 = 2^(-5 - 4)
    r = np.ldexp(np.rint(np.ldexp(x, 4 - e)), e - 4)
    return np.where(np.abs(r) > 448.0, np.nan, r)


# The FP8 P^ V variant rounds P^ (at most 1) as e4m3(2^8 P^) / 2^8, so that P^ in (2^-14, 1] stays
# in E4M3's normal range; V is rounded block by block with a scale taken from the block's largest
# magnitude (see oracle.tiled.tiled_forward, pv="fp8").
P_HAT_FP8_LOG2_SCALE = 8


def fp8_p_hat_round(p, extra=0):
    """P^ as the FP8 P^ V variant feeds it to the product: e4m3(2^(8 + extra) P^) / 2^(8 + extra).

    `extra` (a whole number of binades, broadcast against p; 0 by default) is the variant's own
    range adjustment for rows whose shift leaves every P^ far below 1 (see tiled_forward)."""
    e = (P_HAT_FP8_LOG2_SCALE + np.rint(np.asarray(extra, dtype=np.float64))).astype(np.int64)
    return np.ldexp(e4m3_round(np.ldexp(np.asarray(p, dtype=np.float64), e)), -e)


ELEM_ROUND = {"bf16": bf16_round, "f16": fp16_round, "fp8": fp8_p_hat_round}


def scaled_scores(q_rows, k, scale, mask):
    """S = scale * q k^T for a block of query rows; invisible entries are -inf.

    The attention scores of [FA-backward] §3.1 (softmax(QK^T / sqrt(d_k)) V), with the scale
    passed explicitly.
    """
    s = scale * (q_rows @ k.T)
    return np.where(mask, s, -np.inf)


def row_max_and_repeats(s):
    """rm = rowmax(S) and rs = rowsum(S == rm): the repeated-maximum detection of [BF16-FA] §4.1
    (the same statistic [BF16-FA] §7.1 suggests monitoring).  Visible scores are finite, so a row
    with no visible key is the one whose max is -inf; it gets rs = 0."""
    if s.shape[1] == 0:
        return np.full(s.shape[0], -np.inf), np.zeros(s.shape[0], dtype=np.int64)
    rm = np.max(s, axis=1)
    rs = np.sum(s == rm[:, None], axis=1).astype(np.int64)
    return rm, np.where(rm == -np.inf, 0, rs)


def stable_shift(rm, rs, beta, mode):
    """Row shift m of the safe softmax.

    mode 0: m = rm (the standard safe softmax, [FA-backward] §3.2).
    mode 1: the conditional shift of [BF16-FA] §4.1 / [WhyFail] mechanism 2: with repeated maxima
            (rs > 1), m = beta * rm when rm > 0 and m = 0 when rm < 0; otherwise m = rm.
    mode 2: the same rule with rs replaced by max(rs, 2).
    """
    rm = np.asarray(rm, dtype=np.float64)
    if mode == MODE_STANDARD:
        return rm.copy()
    if mode == MODE_TIE_RULE:
        rep = np.asarray(rs) > 1
    elif mode == MODE_TIE_ANTICIPATE:
        rep = np.ones(rm.shape, dtype=bool)
    else:
        raise ValueError(f"mode must be 0, 1 or 2, got {mode}")
    m = np.where((rm > 0) & rep, beta * rm, rm)
    m = np.where((rm < 0) & rep, 0.0, m)
    return m


@dataclasses.dataclass
class ForwardResult:
    o: np.ndarray  # [N, d] normalised output
    lse: np.ndarray  # [N] natural-log logsumexp of the scaled scores
    rm: np.ndarray  # [N] row max of the scaled scores
    rs: np.ndarray  # [N] number of visible keys attaining the row max (int64)
    m: np.ndarray  # [N] the row shift actually used
    l: np.ndarray  # [N] sum of the unnormalised probabilities exp(S - m)
    ones: np.ndarray  # [N] count of round(exp(S - m)) == 1.0 over visible keys (int64), rounded
    #                  to the 16-bit element type of the P^ V product
    smin: np.ndarray  # [N] row min of the scaled scores over visible keys


def integer_repeat_counts(qi, ki, causal, row_chunk=2048):
    """Row maximum and repeat count (rowsum(S == rowmax(S)), [BF16-FA] §4.1 / §7.1) of the integer
    dot products X = qi ki^T over the visible keys, for integer-valued arrays qi [Nq, d] and
    ki [Nk, d].  Returns (xmax, count) as int64 arrays; a row with no visible key gets count 0.

    The repeat count of the scaled scores S = scale q k^T equals that of X whenever q and k are
    the integer arrays times a common positive factor (grid inputs: entries multiples of 0.5, so
    qi = 2q, ki = 2k), since a positive factor preserves order and equality.  The product is
    formed with a float32 matrix multiply, which is exact here: every partial sum is an integer of
    magnitude at most d max|qi| max|ki|, checked to be below 2^24.  Rows are processed in chunks
    of row_chunk to bound memory."""
    qi = np.asarray(qi)
    ki = np.asarray(ki)
    if not (np.array_equal(qi, np.rint(qi)) and np.array_equal(ki, np.rint(ki))):
        raise ValueError("integer_repeat_counts needs integer-valued inputs")
    bound = qi.shape[1] * (np.abs(qi).max(initial=0)) * (np.abs(ki).max(initial=0))
    if bound >= 2**24:
        raise ValueError("dot products could exceed the exactly representable fp32 integers")
    n, nk = qi.shape[0], ki.shape[0]
    q32 = qi.astype(np.float32)
    k32 = ki.astype(np.float32)
    xmax = np.zeros(n, dtype=np.int64)
    count = np.zeros(n, dtype=np.int64)
    for r0 in range(0, n, row_chunk):
        rows = np.arange(r0, min(n, r0 + row_chunk))
        mask = visible(rows, nk, causal, n)
        x = np.where(mask, q32[rows] @ k32.T, -np.inf)
        mx = x.max(axis=1, initial=-np.inf)
        cnt = np.sum(x == mx[:, None], axis=1)
        live = mx > -np.inf
        xmax[rows] = np.where(live, mx, 0).astype(np.int64)
        count[rows] = np.where(live, cnt, 0)
    return xmax, count


def forward_rows(q, k, v, rows, causal, scale, beta=1.25, mode=MODE_STANDARD, elem="bf16"):
    """The forward of one head for the query rows `rows` (absolute indices into q; the causal mask
    uses them), evaluated without tiling: P_hat = exp(S - m), l = rowsum(P_hat),
    O = diag(l)^-1 P_hat V and LSE = m + ln l ([BF16-FA] §2.1, [FA-practice] §3.3,
    [FA-backward] §2).  `elem` ("bf16" or "f16") is the 16-bit type P^ is rounded to for the
    P^ V product ([FA-practice] §3.2 names both); it only affects the exact-1.0 count.  Returns a
    ForwardResult whose arrays are indexed like `rows`."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows)
    mask = visible(rows, k.shape[0], causal, q.shape[0])
    s = scaled_scores(q[rows], k, scale, mask)
    rm, rs = row_max_and_repeats(s)
    # A row with no visible key (bottom-right alignment with more queries than keys, or no keys)
    # has the empty sum l = 0: O = 0 and LSE = ln 0 = -inf.  No shift applies to it; 0 is stored.
    live = rm > -np.inf
    m = np.where(live, stable_shift(np.where(live, rm, 0.0), rs, beta, mode), 0.0)
    p_hat = np.exp(s - m[:, None])  # exp(-inf) = 0 on invisible keys
    l = p_hat.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(live[:, None], (p_hat @ v) / l[:, None], 0.0)
        lse = np.where(live, m + np.log(l), -np.inf)
    ones = np.sum((ELEM_ROUND[elem](p_hat) == 1.0) & mask, axis=1)
    # The range of the softmax input, to be monitored ([FA-practice] §5): min over visible keys
    # (+inf for a row with none, the min of the empty set).
    smin = np.min(np.where(mask, s, np.inf), axis=1, initial=np.inf)
    return ForwardResult(o, lse, rm, rs, m, l, ones, smin)


def forward(q, k, v, causal, scale, beta=1.25, mode=MODE_STANDARD, row_chunk=1024, elem="bf16"):
    """One head of attention: q [Nq, d], k [Nk, d], v [Nk, d] (float64): forward_rows over all
    rows, in chunks of row_chunk rows to bound memory."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    rm_all = np.zeros(n)
    rs_all = np.zeros(n, dtype=np.int64)
    m_all = np.zeros(n)
    l_all = np.zeros(n)
    ones = np.zeros(n, dtype=np.int64)
    smin = np.zeros(n)
    for r0 in range(0, n, row_chunk):
        rows = np.arange(r0, min(n, r0 + row_chunk))
        fr = forward_rows(q, k, v, rows, causal, scale, beta, mode, elem)
        o[rows], lse[rows] = fr.o, fr.lse
        rm_all[rows], rs_all[rows], m_all[rows], l_all[rows], ones[rows] = fr.rm, fr.rs, fr.m, fr.l, fr.ones
        smin[rows] = fr.smin
    return ForwardResult(o, lse, rm_all, rs_all, m_all, l_all, ones, smin)


def probabilities(q_rows, k, scale, lse_rows, mask):
    """Normalised P = exp(S - LSE) for a block of rows: the recomputation of [FA-backward] §2.
    Invisible entries are 0 (also in a row with no visible key, whose LSE is -inf)."""
    s = scaled_scores(q_rows, k, scale, mask)
    with np.errstate(invalid="ignore"):
        return np.where(mask, np.exp(s - lse_rows[:, None]), 0.0)


@dataclasses.dataclass
class BackwardResult:
    dq: np.ndarray
    dk: np.ndarray
    dv: np.ndarray
    delta: np.ndarray  # [N] rowsum(dO * O)


def backward(q, k, v, do, causal, scale, o=None, lse=None, row_chunk=1024):
    """Gradients of sum(dO * O) with respect to q, k, v for one head.

    The backward by recomputation of [FA-backward] §2 with the preprocessing term
    delta = rowsum(dO o O) of [BF16-FA] §3.1.  With P = softmax(S) and S = scale * q k^T:
      dV = P^T dO,   dP = dO V^T,   dS = P o (dP - delta),
      dQ = scale * dS K,   dK = scale * dS^T Q.
    O and LSE are this oracle's own forward results unless given.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    if o is None or lse is None:
        fr = forward(q, k, v, causal, scale, row_chunk=row_chunk)
        o, lse = fr.o, fr.lse
    n = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.sum(do * o, axis=1)
    for r0 in range(0, n, row_chunk):
        rows = np.arange(r0, min(n, r0 + row_chunk))
        p, ds = _grad_rows(q, k, v, do, rows, causal, scale, lse[rows], delta[rows])
        dv += p.T @ do[rows]
        dq[rows] = scale * (ds @ k)
        dk += scale * (ds.T @ q[rows])
    return BackwardResult(dq, dk, dv, delta)


def _grad_rows(q, k, v, do, rows, causal, scale, lse_rows, delta_rows):
    """P and dS = P o (dP - delta), dP = dO V^T, for the query rows `rows` ([FA-backward] §2,
    [BF16-FA] §3.1)."""
    mask = visible(rows, k.shape[0], causal, q.shape[0])
    p = probabilities(q[rows], k, scale, lse_rows, mask)
    dp = do[rows] @ v.T
    ds = p * (dp - delta_rows[:, None])
    return p, ds


def dq_rows(q, k, v, do, rows, causal, scale, beta=1.25, mode=MODE_STANDARD):
    """dQ and delta of one head for the query rows `rows` alone: each needs only its own row's
    O and LSE (forward_rows) and all keys, so it can be evaluated at any sequence length.
    Returns (dq [len(rows), d], delta [len(rows)])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    rows = np.asarray(rows)
    fr = forward_rows(q, k, v, rows, causal, scale, beta, mode)
    delta = np.sum(do[rows] * fr.o, axis=1)
    _, ds = _grad_rows(q, k, v, do, rows, causal, scale, fr.lse, delta)
    return scale * (ds @ k), delta


def exact_causal_pairs(N):
    return N * (N + 1) // 2


def visible_pairs(Nq, Nk, causal):
    """Number of (query, key) pairs visible under the mask `visible` defines, by summing the
    per-row counts: min(Nk, max(0, i + off + 1)) for a causal alignment with offset off."""
    causal = int(causal)
    if causal == CAUSAL_NONE:
        return Nq * Nk
    off = 0 if causal == CAUSAL_TOP_LEFT else Nk - Nq
    return sum(min(Nk, max(0, i + off + 1)) for i in range(Nq))

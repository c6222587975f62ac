"""fp64 replay of the tiled online-softmax forward, with the per-tile stabilised shift.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the CPU-baseline leg of
the benchmark may import this module; the HIP library never calls it.

It follows the online softmax of the BF16 Flash Attention article at ijyty.com/news/896914, §2.1,
step by step over key blocks of width `bc` (all query rows at once, in float64):

    m   = shift(running max, running repeat count)
    P^  = exp(S - m)
    l   = exp(m_prev - m) * l_prev + rowsum(P^)
    O   = diag(exp(m_prev - m)) O_prev + P^ V
and at the end O = diag(l)^-1 O, LSE = m + ln l.

The pages do not say how repeated maxima are counted across blocks.  The reading taken here:
the block maximum tm and its count tc are merged into a running (r, c) by
    r' = max(r, tm),   c' = [tm == r'] tc + [r == r'] c,
so after the last block c equals the untiled count, and the shift of §4.1 is applied per block
from the running (r, c).  With the tie-conditional rule (mode 1) the first occurrence of a
maximum whose repeat only arrives in a later block is exponentiated with m = r and gives an
unnormalised probability of exactly 1.0; the `ones` output counts those, per row, exactly as a
kernel that processes key blocks in the same order and width would produce them.
"""
from __future__ import annotations

import numpy as np

from .attention import ELEM_ROUND, e4m3_round, fp8_p_hat_round, stable_shift, visible


def fp8_v_block(v_block):
    """V of one key block as the FP8 P^ V variant feeds it to the product: with the block's
    dynamic scale s = amax |V| / 448 (fp32 division; s = 1 for an all-zero block), each entry is
    rounded as e4m3(fp32(v * fp32(1 / s))) and stands for that value times s.  The scale and the
    scaled value are formed in fp32 because that is where the rounding to E4M3 is decided.
    Returns (the dequantised block as float64, s)."""
    vb = np.asarray(v_block, dtype=np.float64)
    amax = np.float32(np.max(np.abs(vb))) if vb.size else np.float32(0.0)
    s = np.float32(amax) / np.float32(448.0) if amax > 0 else np.float32(1.0)
    inv = np.float32(1.0) / s
    scaled = (vb.astype(np.float32) * inv).astype(np.float64)
    return e4m3_round(scaled) * np.float64(s), float(s)


def tiled_forward(q, k, v, causal, scale, beta=1.25, mode=0, bc=64, order=None, elem="bf16",
                  pv="exact"):
    """Tiled forward over one head; returns dict(o, lse, r, c, m, ones).

    `order` lists the key-block indices in processing order (default: ascending).  Key blocks
    entirely invisible to a row leave that row's state unchanged.  `elem` ("bf16", "f16" or "fp8")
    is the type P^ is rounded to for the exact-1.0 count.

    pv="fp8" is the FP8 P^ V variant ([BF16-FA] §6.1 names FP8 as the next lower precision): the
    block's product P^ V takes P^ rounded by fp8_p_hat_round and V rounded by fp8_v_block (one
    dynamic scale per key block of width bc); the row sum l, the shift m and the LSE are the
    unrounded ones, and O = acc / l as before.  Where the shift lies more than 5 binades below the
    running maximum (g = (m - r) / ln 2 > 5), every P^ of the row is below 2^-5 and e4m3(2^8 P^)
    would lose it to the subnormals and to zero; the variant then rounds P^ as
    e4m3(2^(8 + k) P^) / 2^(8 + k) with k = floor(g) - 5, which puts the row's largest value in
    (2^2, 2^3] before rounding.  (The variant's own design: the pages fix no FP8 scaling.  A kernel
    evaluates g in fp32, so for g within rounding of a whole number its k can differ by one; the
    rounding error stays within the same bound.)
    """
    if pv not in ("exact", "fp8"):
        raise ValueError(f"pv must be 'exact' or 'fp8', got {pv!r}")
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    n_keys = k.shape[0]
    n_blocks = -(-n_keys // bc)
    if order is None:
        order = range(n_blocks)
    rows = np.arange(n)
    mask_all = visible(rows, n_keys, causal, n)

    r = np.full(n, -np.inf)
    c = np.zeros(n, dtype=np.int64)
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, v.shape[1]))
    ones = np.zeros(n, dtype=np.int64)
    for j in order:
        k0, k1 = j * bc, min(n_keys, (j + 1) * bc)
        mask = mask_all[:, k0:k1]
        s = np.where(mask, scale * (q @ k[k0:k1].T), -np.inf)
        tm = np.max(s, axis=1)
        tc = np.sum((s == tm[:, None]) & mask, axis=1)
        r_new = np.maximum(r, tm)
        c = np.where(tm == r_new, tc, 0) + np.where(r == r_new, c, 0)
        r = r_new
        live = np.isfinite(r)  # rows that have seen at least one visible key
        m_new = np.where(live, stable_shift(np.where(live, r, 0.0), c, beta, mode), -np.inf)
        alpha = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m, 0.0) - np.where(live, m_new, 0.0)), 0.0)
        p_hat = np.where(mask, np.exp(s - np.where(live, m_new, 0.0)[:, None]), 0.0)
        l = alpha * l + p_hat.sum(axis=1)
        if pv == "fp8":
            gap = np.where(live, (np.where(live, m_new, 0.0) - np.where(live, r, 0.0)) / np.log(2.0), 0.0)
            extra = np.where(gap > 5.0, np.floor(gap) - 5.0, 0.0)
            acc = alpha[:, None] * acc + fp8_p_hat_round(p_hat, extra[:, None]) @ fp8_v_block(v[k0:k1])[0]
        else:
            acc = alpha[:, None] * acc + p_hat @ v[k0:k1]
        ones += np.sum((ELEM_ROUND[elem](p_hat) == 1.0) & mask, axis=1)
        m = m_new
    # A row with no visible key keeps l = 0: O = 0 and LSE = -inf.
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(l[:, None] > 0, acc / l[:, None], 0.0)
        lse = np.where(l > 0, m + np.log(l), -np.inf)
    return {"o": o, "lse": lse, "r": r, "c": c, "m": m, "ones": ones}


def tiled_ones(q, k, causal, scale, beta=1.25, mode=0, bc=64, order=None, elem="bf16"):
    """Per-row count of exact-1.0 bf16 unnormalised probabilities under block-wise processing.

    Same recurrence as tiled_forward without V; used where only the count is needed (large
    heads), to save the P^ V product.  A block invisible to a row leaves that row's state
    unchanged (as in tiled_forward), so each block is evaluated only for the rows that see at
    least one of its keys.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n = q.shape[0]
    n_keys = k.shape[0]
    n_blocks = -(-n_keys // bc)
    if order is None:
        order = range(n_blocks)
    rows_all = np.arange(n)
    r = np.full(n, -np.inf)
    c = np.zeros(n, dtype=np.int64)
    ones = np.zeros(n, dtype=np.int64)
    for j in order:
        k0, k1 = j * bc, min(n_keys, (j + 1) * bc)
        mask = visible(rows_all, n_keys, causal, n, keys=np.arange(k0, k1))
        rows = np.nonzero(mask.any(axis=1))[0]
        mask = mask[rows]
        s = np.where(mask, scale * (q[rows] @ k[k0:k1].T), -np.inf)
        tm = np.max(s, axis=1)
        tc = np.sum((s == tm[:, None]) & mask, axis=1)
        r_new = np.maximum(r[rows], tm)
        c[rows] = np.where(tm == r_new, tc, 0) + np.where(r[rows] == r_new, c[rows], 0)
        r[rows] = r_new
        live = np.isfinite(r_new)
        m = stable_shift(np.where(live, r_new, 0.0), c[rows], beta, mode)
        p_hat = np.where(mask, np.exp(s - m[:, None]), 0.0)
        ones[rows] += np.sum((ELEM_ROUND[elem](p_hat) == 1.0) & mask, axis=1)
    return ones

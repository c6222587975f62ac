"""Seeded 16-bit input generators for the five attention workloads.

Every tensor is drawn on the CPU with a ``torch.Generator`` seeded per workload, as float32,
multiplied by the workload's sigma, and rounded to bfloat16 (default) or float16 by torch's
round-to-nearest-even cast.  Q, K, V and dO are drawn in that order.  The workloads stand in for the attention layers
of the models the pages train (GPT-2 small/medium and LLaMA-7B shapes); no dataset or weight is
involved.

The module contains no softmax, no matmul and no gradient: only random draws and the input
constructions below.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import numpy as np
import torch

# Entries of the tie-heavy grid: exact in bf16 and fp16, and every dot product of two rows of length
# <= 512 drawn from it is an exact multiple of 0.25 in fp32.
GRID_VALUES = (-1.0, -0.5, 0.0, 0.5, 1.0)


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    cid: int
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    scale: float
    modes: tuple
    seed: int
    sigma_qk: float = 1.0
    kind: str = "randn"  # "randn" | "dup" | "sink" | "grid"

    def with_shape(self, **kw) -> "WorkloadConfig":
        return dataclasses.replace(self, **kw)


def _inv_sqrt_f32(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))


CONFIGS = {
    1: WorkloadConfig(1, "tiny-dup", 1, 1, 128, 64, False, 0.125, (0, 1, 2), 1001, kind="dup"),
    2: WorkloadConfig(2, "gpt2-small", 8, 12, 1024, 64, True, 0.125, (1, 2), 1002),
    3: WorkloadConfig(3, "gpt2-medium-sink", 4, 16, 2048, 64, True, 0.125, (0, 1, 2), 1003,
                      sigma_qk=3.0, kind="sink"),
    4: WorkloadConfig(4, "llama7b", 1, 32, 8192, 128, True, _inv_sqrt_f32(128), (1, 2), 1004),
    5: WorkloadConfig(5, "long-tie-grid", 1, 32, 16384, 128, True, _inv_sqrt_f32(128), (1, 2), 1005,
                      kind="grid"),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _randn16(g: torch.Generator, shape, sigma: float = 1.0, dtype=torch.bfloat16) -> torch.Tensor:
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if sigma != 1.0:
        x = x * sigma
    return x.to(dtype)


def _grid16(g: torch.Generator, shape, dtype=torch.bfloat16) -> torch.Tensor:
    idx = torch.randint(0, len(GRID_VALUES), shape, generator=g)
    table = torch.tensor(GRID_VALUES, dtype=torch.float32)
    return table[idx].to(dtype)


def randn_inputs(B, H, N, d, seed, sigma_qk=1.0, dtype=torch.bfloat16):
    """Q, K ~ N(0, sigma_qk^2), V, dO ~ N(0, 1); `dtype` (bf16 or fp16), shape [B, H, N, d]."""
    g = _gen(seed)
    shape = (B, H, N, d)
    q = _randn16(g, shape, sigma_qk, dtype)
    k = _randn16(g, shape, sigma_qk, dtype)
    v = _randn16(g, shape, 1.0, dtype)
    do = _randn16(g, shape, 1.0, dtype)
    return {"q": q, "k": k, "v": v, "do": do}


def rect_inputs(B, H, Nq, Nk, d, seed, grid=False, dtype=torch.bfloat16):
    """Q and dO [B, H, Nq, d], K and V [B, H, Nk, d] for a query block attending to a key sequence
    of another length (drawn in the order Q, K, V, dO).  Q, K ~ N(0, 1), or uniform over
    GRID_VALUES with grid=True; V, dO ~ N(0, 1)."""
    g = _gen(seed)
    qs, ks = (B, H, Nq, d), (B, H, Nk, d)
    if grid:
        q = _grid16(g, qs, dtype)
        k = _grid16(g, ks, dtype)
    else:
        q = _randn16(g, qs, 1.0, dtype)
        k = _randn16(g, ks, 1.0, dtype)
    v = _randn16(g, ks, 1.0, dtype)
    do = _randn16(g, qs, 1.0, dtype)
    return {"q": q, "k": k, "v": v, "do": do}


def grid_inputs(B, H, N, d, seed, dtype=torch.bfloat16):
    """Q, K uniform over GRID_VALUES (exact ties in row maxima are frequent); V, dO ~ N(0, 1)."""
    g = _gen(seed)
    shape = (B, H, N, d)
    q = _grid16(g, shape, dtype)
    k = _grid16(g, shape, dtype)
    v = _randn16(g, shape, 1.0, dtype)
    do = _randn16(g, shape, 1.0, dtype)
    return {"q": q, "k": k, "v": v, "do": do}


def tied_maxima_inputs(N, d, seed, dtype=torch.bfloat16, tie_keys=(7, 200), c=2.0, n=None):
    """One head ([1, 1, N, d]) whose query rows include constructed repeated maxima of chosen sign.

    The first 3n coordinates are split into three blocks P = [0, n), M = [n, 2n), Z = [2n, 3n)
    (n = d // 3 - 1 by default).  The keys in `tie_keys` hold c on P, c on M and 0 on Z (0 on the
    remaining coordinates); every other key holds grid values {-0.5, -0.25, 0, 0.25, 0.5} on P,
    c + 0.5 + {0, 0.25, 0.5} on M and on Z, and N(0, 1) draws elsewhere.  Constructed queries:
      pos:     a c on P (a in 1/4, 1, 4, 8), 0 elsewhere: the tie keys give the maximum a n c^2
               and every other key at most a c (n/2) < a n c^2;
      neg:     -a c on M: the tie keys give -a n c^2, every other key less (its M entries exceed c);
      zero:    -a c on Z: the tie keys give exactly 0, every other key less;
      allzero: all coordinates 0: every key gives 0 (the whole row ties).
    All these dot products are exact in fp32 (entries are multiples of 1/4 with few significant
    bits), so the row maximum is attained exactly by the tie keys.  Every other query row is
    N(0, 1/16).  V and dO are N(0, 1).  The constructed rows sit in the first and last 256-row
    query tiles.  Returns (tensors, rows) with rows a dict of lists of row indices per kind."""
    n = d // 3 - 1 if n is None else n
    if 3 * n > d or max(tie_keys) >= N or N < 300:
        raise ValueError("shape too small for the construction")
    g = _gen(seed)
    q = 0.25 * torch.randn((N, d), generator=g)
    k = torch.randn((N, d), generator=g)
    v = torch.randn((N, d), generator=g)
    do = torch.randn((N, d), generator=g)
    grid_p = torch.tensor((-0.5, -0.25, 0.0, 0.25, 0.5))[torch.randint(0, 5, (N, n), generator=g)]
    grid_m = torch.tensor((0.0, 0.25, 0.5))[torch.randint(0, 3, (N, n), generator=g)]
    grid_z = torch.tensor((0.0, 0.25, 0.5))[torch.randint(0, 3, (N, n), generator=g)]
    k[:, 0:n] = grid_p
    k[:, n:2 * n] = c + 0.5 + grid_m
    k[:, 2 * n:3 * n] = c + 0.5 + grid_z
    for j in tie_keys:
        k[j] = 0.0
        k[j, 0:2 * n] = c
    mults = (0.25, 1.0, 4.0, 8.0)
    base = (10, N - 40)
    rows = {"pos": [], "neg": [], "zero": [], "allzero": []}
    for b0 in base:
        for i, a in enumerate(mults):
            for kind, lo, sign, off in (("pos", 0, 1.0, 0), ("neg", n, -1.0, 4), ("zero", 2 * n, -1.0, 8)):
                r = b0 + off + i
                q[r] = 0.0
                q[r, lo:lo + n] = sign * a * c
                rows[kind].append(r)
        q[b0 + 12] = 0.0
        rows["allzero"].append(b0 + 12)
    t = {"q": q, "k": k, "v": v, "do": do}
    return {n_: x_.reshape(1, 1, N, d).to(dtype) for n_, x_ in t.items()}, rows


def _apply_dup(t):
    """Key 17 := key 3 and queries 0..7 := key 3, so rows 0..7 carry an exact repeated maximum."""
    k, q = t["k"], t["q"]
    k[:, :, 17, :] = k[:, :, 3, :]
    n_rows = min(8, q.shape[2])
    q[:, :, :n_rows, :] = k[:, :, 3:4, :].expand(-1, -1, n_rows, -1)
    return t


def _apply_sink(t):
    """Key 0 of each (b, h) := 4 * u rounded to the tensors' type, u = the mean query direction
    normalised to unit length."""
    q, k = t["q"], t["k"]
    qm = q.to(torch.float64).mean(dim=2)  # [B, H, d]
    u = qm / qm.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    k[:, :, 0, :] = (4.0 * u).to(k.dtype)
    return t


def make_inputs(cfg, dtype=torch.bfloat16, **overrides):
    """Inputs for a workload (a WorkloadConfig or its id) in `dtype` (bf16 or fp16); keyword
    overrides replace B/H/N/d/seed."""
    if not isinstance(cfg, WorkloadConfig):
        cfg = CONFIGS[int(cfg)]
    if overrides:
        cfg = cfg.with_shape(**overrides)
    if cfg.kind == "grid":
        t = grid_inputs(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed, dtype)
    else:
        t = randn_inputs(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed, cfg.sigma_qk, dtype)
    if cfg.kind == "dup":
        t = _apply_dup(t)
    elif cfg.kind == "sink":
        t = _apply_sink(t)
    return t


def tensor_digest(t: torch.Tensor) -> str:
    """SHA-256 of a tensor's raw bytes (16-bit float tensors are hashed through their int16 view)."""
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.view(torch.int16)
    return hashlib.sha256(t.contiguous().numpy().tobytes()).hexdigest()

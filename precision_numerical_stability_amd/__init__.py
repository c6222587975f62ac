"""BF16 (and FP16) FlashAttention forward/backward for MI355X (gfx950) with the stabilised softmax
shift.

Thin Python binding over the C ABI of libfa_stable.so (include/fa_stable.h).  The functions named
like the C entry points (fa_fwd, fa_fwd_ex, fa_bwd, ...) only marshal torch tensors into
pointers and sizes; every step of the computation runs in the library's HIP kernels.  torch
provides device memory and streams.

The saved state of the autograd wrapper is q, k, v, o and lse; the backward recomputes the
probabilities.  Do not wrap `attention` in torch.utils.checkpoint: the backward already
recomputes the forward's work, and an outer checkpoint would run it again ("FlashAttention
训练时为什么会梯度爆炸", cnnetsun.cn/a/2497354, §4).
"""
from __future__ import annotations

import ctypes
import math

import torch  # loaded first so that its HIP runtime is the one this library binds to

from . import _ffi
from ._ffi import (FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_HEADDIM, FA_ERR_PARAM, FA_ERR_ALIGN,
                   FA_ERR_HIP, FA_ERR_SCRATCH, FA_BWD_DELTA, FA_BWD_DKDV, FA_BWD_DQ, FA_BWD_ALL,
                   FA_FWD_COMPENSATED_SUM, FA_CAUSAL_NONE, FA_CAUSAL_TOP_LEFT,
                   FA_CAUSAL_BOTTOM_RIGHT, FA_ELEM_BF16, FA_ELEM_F16)

_lib = _ffi.load_library()

_runtimes = _ffi.hip_runtimes_mapped()
if len(_runtimes) > 1:
    raise ImportError(f"more than one HIP runtime is mapped into this process: {_runtimes}")

STANDARD = 0
TIE_RULE = 1
TIE_ANTICIPATE = 2
DEFAULT_BETA = 1.25

__all__ = [
    "fa_fwd", "fa_fwd_ex", "fa_fwd_stats", "fa_fwd_qk", "fa_fwd_elem", "FA_FWD_COMPENSATED_SUM",
    "fa_bwd", "fa_bwd_ex", "fa_bwd_qk", "fa_bwd_elem", "FA_ELEM_BF16", "FA_ELEM_F16",
    "fa_fwd_fp8pv", "fa_fwd_fp8pv_workspace_bytes", "forward_fp8pv",
    "fa_bwd_workspace_bytes", "fa_fwd_kv_block", "fa_fwd_diag", "fa_bwd_noalloc",
    "fa_bwd_noalloc_max_rows",
    "FA_CAUSAL_NONE", "FA_CAUSAL_TOP_LEFT", "FA_CAUSAL_BOTTOM_RIGHT", "fa_status_str",
    "fa_last_hip_error", "FaError", "forward", "backward", "attention", "STANDARD", "TIE_RULE",
    "TIE_ANTICIPATE", "DEFAULT_BETA", "library_path",
]


class FaError(RuntimeError):
    def __init__(self, status: int):
        msg = fa_status_str(status)
        if status == FA_ERR_HIP:
            msg += f" (hipError_t {fa_last_hip_error()})"
        super().__init__(msg)
        self.status = status


def library_path() -> str:
    return _ffi.LIB_PATH


def fa_status_str(status: int) -> str:
    return _lib.fa_status_str(int(status)).decode()


def fa_last_hip_error() -> int:
    return int(_lib.fa_last_hip_error())


def fa_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(_lib.fa_bwd_workspace_bytes(B, H, N, d))


def fa_fwd_kv_block(d: int, causal: bool) -> int:
    return int(_lib.fa_fwd_kv_block(d, int(bool(causal))))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream_handle(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _raise(status):
    if status != FA_OK:
        raise FaError(status)


def fa_fwd_ex(q, k, v, o, lse, dupcnt, ones, causal, scale, beta, stable_flag, stream=None):
    """Call fa_fwd_ex on torch tensors: q, k, v, o [B,H,N,d] bf16, lse [B,H,N] fp32, dupcnt and
    ones [B,H,N] int32 or None.  Launches on `stream` (default: the current stream)."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check(t, name, torch.bfloat16, (B, H, N, d))
    _check(lse, "lse", torch.float32, (B, H, N))
    for name, t in (("dupcnt", dupcnt), ("ones", ones)):
        if t is not None:
            _check(t, name, torch.int32, (B, H, N))
    st = _lib.fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dupcnt), _ptr(ones),
                        B, H, N, d, int(causal), float(scale), float(beta), int(stable_flag),
                        _stream_handle(q.device, stream))
    _raise(st)


def fa_fwd_stats(q, k, v, o, lse, dupcnt, ones, smin, smax, causal, scale, beta, stable_flag,
                 flags=0, stream=None):
    """Call fa_fwd_stats on torch tensors: as fa_fwd_ex, plus smin and smax [B,H,N] fp32 or None
    (per-row min and max of the scaled visible scores) and flags (FA_FWD_COMPENSATED_SUM)."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check(t, name, torch.bfloat16, (B, H, N, d))
    _check(lse, "lse", torch.float32, (B, H, N))
    for name, t in (("dupcnt", dupcnt), ("ones", ones)):
        if t is not None:
            _check(t, name, torch.int32, (B, H, N))
    for name, t in (("smin", smin), ("smax", smax)):
        if t is not None:
            _check(t, name, torch.float32, (B, H, N))
    st = _lib.fa_fwd_stats(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dupcnt), _ptr(ones),
                           _ptr(smin), _ptr(smax), B, H, N, d, int(causal), float(scale), float(beta),
                           int(stable_flag), int(flags), _stream_handle(q.device, stream))
    _raise(st)


def fa_fwd_qk(q, k, v, o, lse, dupcnt, ones, smin, smax, causal, scale, beta, stable_flag,
              flags=0, stream=None):
    """Call fa_fwd_qk on torch tensors: q, o [B,H,Nq,d] and k, v [B,H,Nk,d] bf16; lse and the
    optional diagnostics [B,H,Nq]; causal 0 (none), 1 (top-left) or 2 (bottom-right)."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    for name, t, n in (("q", q, Nq), ("o", o, Nq), ("k", k, Nk), ("v", v, Nk)):
        _check(t, name, torch.bfloat16, (B, H, n, d))
    _check(lse, "lse", torch.float32, (B, H, Nq))
    for name, t, dt in (("dupcnt", dupcnt, torch.int32), ("ones", ones, torch.int32),
                        ("smin", smin, torch.float32), ("smax", smax, torch.float32)):
        if t is not None:
            _check(t, name, dt, (B, H, Nq))
    st = _lib.fa_fwd_qk(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dupcnt), _ptr(ones),
                        _ptr(smin), _ptr(smax), B, H, Nq, Nk, d, int(causal), float(scale),
                        float(beta), int(stable_flag), int(flags), _stream_handle(q.device, stream))
    _raise(st)


_ELEM_OF_DTYPE = {torch.bfloat16: FA_ELEM_BF16, torch.float16: FA_ELEM_F16}


def _elem(t, name):
    if t.dtype not in _ELEM_OF_DTYPE:
        raise ValueError(f"{name} must be bfloat16 or float16, got {t.dtype}")
    return _ELEM_OF_DTYPE[t.dtype]


def fa_fwd_elem(q, k, v, o, lse, dupcnt, ones, smin, smax, causal, scale, beta, stable_flag,
                flags=0, stream=None):
    """Call fa_fwd_elem on torch tensors: as fa_fwd_qk, with q, k, v, o all bfloat16 or all
    float16 (the element type is taken from q)."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    elem = _elem(q, "q")
    for name, t, n in (("q", q, Nq), ("o", o, Nq), ("k", k, Nk), ("v", v, Nk)):
        _check(t, name, q.dtype, (B, H, n, d))
    _check(lse, "lse", torch.float32, (B, H, Nq))
    for name, t, dt in (("dupcnt", dupcnt, torch.int32), ("ones", ones, torch.int32),
                        ("smin", smin, torch.float32), ("smax", smax, torch.float32)):
        if t is not None:
            _check(t, name, dt, (B, H, Nq))
    st = _lib.fa_fwd_elem(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dupcnt), _ptr(ones),
                          _ptr(smin), _ptr(smax), B, H, Nq, Nk, d, int(causal), float(scale),
                          float(beta), int(stable_flag), int(flags), elem,
                          _stream_handle(q.device, stream))
    _raise(st)


def fa_fwd_diag(q, k, v, o, lse, dupcnt, ones, smin, smax, mshift, causal, scale, beta, stable_flag,
                flags=0, stream=None):
    """Call fa_fwd_diag on torch tensors: as fa_fwd_elem, plus mshift [B,H,Nq] fp32 or None (the
    per-row shift of the repeated-maximum rule after the last key block)."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    elem = _elem(q, "q")
    for name, t, n in (("q", q, Nq), ("o", o, Nq), ("k", k, Nk), ("v", v, Nk)):
        _check(t, name, q.dtype, (B, H, n, d))
    _check(lse, "lse", torch.float32, (B, H, Nq))
    for name, t, dt in (("dupcnt", dupcnt, torch.int32), ("ones", ones, torch.int32),
                        ("smin", smin, torch.float32), ("smax", smax, torch.float32),
                        ("mshift", mshift, torch.float32)):
        if t is not None:
            _check(t, name, dt, (B, H, Nq))
    st = _lib.fa_fwd_diag(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dupcnt), _ptr(ones),
                          _ptr(smin), _ptr(smax), _ptr(mshift), B, H, Nq, Nk, d, int(causal),
                          float(scale), float(beta), int(stable_flag), int(flags), elem,
                          _stream_handle(q.device, stream))
    _raise(st)


def fa_fwd_fp8pv_workspace_bytes(B: int, H: int, Nk: int, d: int) -> int:
    return int(_lib.fa_fwd_fp8pv_workspace_bytes(B, H, Nk, d))


def fa_fwd_fp8pv(q, k, v, o, lse, dupcnt, ones, smin, smax, workspace, causal, scale, beta,
                 stable_flag, flags=0, stream=None):
    """Call fa_fwd_fp8pv on torch tensors: as fa_fwd_qk (bf16), plus `workspace`, a uint8 CUDA
    tensor of at least fa_fwd_fp8pv_workspace_bytes(B, H, Nk, d) bytes."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    for name, t, n in (("q", q, Nq), ("o", o, Nq), ("k", k, Nk), ("v", v, Nk)):
        _check(t, name, torch.bfloat16, (B, H, n, d))
    _check(lse, "lse", torch.float32, (B, H, Nq))
    for name, t, dt in (("dupcnt", dupcnt, torch.int32), ("ones", ones, torch.int32),
                        ("smin", smin, torch.float32), ("smax", smax, torch.float32)):
        if t is not None:
            _check(t, name, dt, (B, H, Nq))
    need = fa_fwd_fp8pv_workspace_bytes(B, H, Nk, d)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or workspace.numel() < need:
        raise ValueError(f"workspace must be a uint8 CUDA tensor of at least {need} bytes")
    st = _lib.fa_fwd_fp8pv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dupcnt), _ptr(ones),
                           _ptr(smin), _ptr(smax), _ptr(workspace), B, H, Nq, Nk, d, int(causal),
                           float(scale), float(beta), int(stable_flag), int(flags),
                           _stream_handle(q.device, stream))
    _raise(st)


def fa_fwd(q, k, v, o, lse, causal, scale, beta, stable_flag, stream=None):
    fa_fwd_ex(q, k, v, o, lse, None, None, causal, scale, beta, stable_flag, stream)


def fa_bwd_ex(q, k, v, o, lse, dO, dq, dk, dv, delta_ws, causal, scale, beta=DEFAULT_BETA,
              stable_flag=STANDARD, stages=_ffi.FA_BWD_ALL, stream=None):
    """Call fa_bwd_ex on torch tensors (shapes as in fa_fwd_ex; delta_ws fp32 [B,H,N]); `stages`
    is a mask of FA_BWD_DELTA, FA_BWD_DKDV and FA_BWD_DQ."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dO", dO), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        _check(t, name, torch.bfloat16, (B, H, N, d))
    _check(lse, "lse", torch.float32, (B, H, N))
    _check(delta_ws, "delta_ws", torch.float32, (B, H, N))
    st = _lib.fa_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
                        _ptr(dk), _ptr(dv), _ptr(delta_ws), B, H, N, d, int(causal), float(scale),
                        float(beta), int(stable_flag), int(stages), _stream_handle(q.device, stream))
    _raise(st)


def fa_bwd_qk(q, k, v, o, lse, dO, dq, dk, dv, delta_ws, causal, scale, beta=DEFAULT_BETA,
              stable_flag=STANDARD, stages=_ffi.FA_BWD_ALL, stream=None):
    """Call fa_bwd_qk on torch tensors: q, o, dO, dq [B,H,Nq,d] and k, v, dk, dv [B,H,Nk,d] bf16;
    lse and delta_ws fp32 [B,H,Nq]; causal 0, 1 or 2 as in fa_fwd_qk."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    for name, t, n in (("q", q, Nq), ("o", o, Nq), ("dO", dO, Nq), ("dq", dq, Nq), ("k", k, Nk),
                       ("v", v, Nk), ("dk", dk, Nk), ("dv", dv, Nk)):
        _check(t, name, torch.bfloat16, (B, H, n, d))
    _check(lse, "lse", torch.float32, (B, H, Nq))
    _check(delta_ws, "delta_ws", torch.float32, (B, H, Nq))
    st = _lib.fa_bwd_qk(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
                        _ptr(dk), _ptr(dv), _ptr(delta_ws), B, H, Nq, Nk, d, int(causal),
                        float(scale), float(beta), int(stable_flag), int(stages),
                        _stream_handle(q.device, stream))
    _raise(st)


def fa_bwd_elem(q, k, v, o, lse, dO, dq, dk, dv, delta_ws, causal, scale, beta=DEFAULT_BETA,
                stable_flag=STANDARD, stages=_ffi.FA_BWD_ALL, stream=None):
    """Call fa_bwd_elem on torch tensors: as fa_bwd_qk, with every 16-bit tensor bfloat16 or every
    one float16 (the element type is taken from q)."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    elem = _elem(q, "q")
    for name, t, n in (("q", q, Nq), ("o", o, Nq), ("dO", dO, Nq), ("dq", dq, Nq), ("k", k, Nk),
                       ("v", v, Nk), ("dk", dk, Nk), ("dv", dv, Nk)):
        _check(t, name, q.dtype, (B, H, n, d))
    _check(lse, "lse", torch.float32, (B, H, Nq))
    _check(delta_ws, "delta_ws", torch.float32, (B, H, Nq))
    st = _lib.fa_bwd_elem(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
                          _ptr(dk), _ptr(dv), _ptr(delta_ws), B, H, Nq, Nk, d, int(causal),
                          float(scale), float(beta), int(stable_flag), int(stages), elem,
                          _stream_handle(q.device, stream))
    _raise(st)


def fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, delta_ws, causal, scale, beta=DEFAULT_BETA,
           stable_flag=STANDARD, stream=None):
    """Call fa_bwd on torch tensors (shapes as in fa_fwd_ex; delta_ws fp32 [B,H,N])."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dO", dO), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        _check(t, name, torch.bfloat16, (B, H, N, d))
    _check(lse, "lse", torch.float32, (B, H, N))
    _check(delta_ws, "delta_ws", torch.float32, (B, H, N))
    st = _lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk),
                     _ptr(dv), _ptr(delta_ws), B, H, N, d, int(causal), float(scale), float(beta),
                     int(stable_flag), _stream_handle(q.device, stream))
    _raise(st)


def fa_bwd_noalloc_max_rows() -> int:
    return int(_lib.fa_bwd_noalloc_max_rows())


def fa_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, causal, scale, beta=DEFAULT_BETA,
                   stable_flag=STANDARD, stream=None):
    """Call fa_bwd_noalloc on torch tensors (shapes as fa_bwd, no delta workspace): the backward
    for callers that cannot allocate; delta lives in the library's per-GPU scratch."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dO", dO), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        _check(t, name, torch.bfloat16, (B, H, N, d))
    _check(lse, "lse", torch.float32, (B, H, N))
    st = _lib.fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
                             _ptr(dk), _ptr(dv), B, H, N, d, int(causal), float(scale), float(beta),
                             int(stable_flag), _stream_handle(q.device, stream))
    _raise(st)


def _default_scale(d):
    return 1.0 / math.sqrt(d)


def forward(q, k, v, causal=False, scale=None, beta=DEFAULT_BETA, stable_flag=TIE_RULE,
            stats=False, monitor=False, compensated_sum=False, shift=False, stream=None):
    """Allocate outputs and run the forward (fa_fwd_diag: bfloat16 or float16 tensors; k and v may
    hold a different number of keys than q has queries; causal 0/False, 1/True (top-left) or 2
    (bottom-right)).  Returns
    (o, lse), plus (dupcnt, ones) with stats=True, plus (smin, smax) with monitor=True, plus the
    per-row shift m with shift=True.  compensated_sum selects the Kahan row sum."""
    B, H, N, d = q.shape
    scale = _default_scale(d) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    dup = ones = smin = smax = None
    if stats:
        dup = torch.empty((B, H, N), dtype=torch.int32, device=q.device)
        ones = torch.empty((B, H, N), dtype=torch.int32, device=q.device)
    if monitor:
        smin = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        smax = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    msh = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if shift else None
    flags = FA_FWD_COMPENSATED_SUM if compensated_sum else 0
    fa_fwd_diag(q, k, v, o, lse, dup, ones, smin, smax, msh, int(causal), scale, beta, stable_flag,
                flags, stream)
    out = (o, lse)
    if stats:
        out += (dup, ones)
    if monitor:
        out += (smin, smax)
    if shift:
        out += (msh,)
    return out


def forward_fp8pv(q, k, v, causal=False, scale=None, beta=DEFAULT_BETA, stable_flag=TIE_RULE,
                  stats=False, monitor=False, compensated_sum=False, stream=None):
    """As forward() for bf16 tensors, with the P^ V product in FP8 (fa_fwd_fp8pv); allocates the
    workspace with torch."""
    B, H, N, d = q.shape
    scale = _default_scale(d) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(1, fa_fwd_fp8pv_workspace_bytes(B, H, k.shape[2], d)), dtype=torch.uint8,
                     device=q.device)
    dup = ones = smin = smax = None
    if stats:
        dup = torch.empty((B, H, N), dtype=torch.int32, device=q.device)
        ones = torch.empty((B, H, N), dtype=torch.int32, device=q.device)
    if monitor:
        smin = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        smax = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    flags = FA_FWD_COMPENSATED_SUM if compensated_sum else 0
    fa_fwd_fp8pv(q, k, v, o, lse, dup, ones, smin, smax, ws, int(causal), scale, beta, stable_flag,
                 flags, stream)
    out = (o, lse)
    if stats:
        out += (dup, ones)
    if monitor:
        out += (smin, smax)
    return out


def backward(q, k, v, o, lse, dO, causal=False, scale=None, stream=None):
    """Allocate gradients and workspace and run the backward (fa_bwd_elem).  Returns (dq, dk, dv)."""
    B, H, N, d = q.shape
    scale = _default_scale(d) if scale is None else scale
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_bwd_elem(q, k, v, o, lse, dO, dq, dk, dv, delta, int(causal), scale, stream=stream)
    return dq, dk, dv


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, scale, beta, stable_flag):
        o, lse = forward(q, k, v, causal, scale, beta, stable_flag)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal = causal
        ctx.scale = scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = backward(q, k, v, o, lse, do.contiguous(), ctx.causal, ctx.scale)
        return dq, dk, dv, None, None, None, None


def attention(q, k, v, causal=False, scale=None, beta=DEFAULT_BETA, stable_flag=TIE_RULE):
    """Differentiable attention on bfloat16 or float16 GPU tensors q [B,H,Nq,d], k and v [B,H,Nk,d]
    (d = 64 or 128); causal 0/False, 1/True (top-left) or 2 (bottom-right)."""
    scale = _default_scale(q.shape[-1]) if scale is None else scale
    return _Attention.apply(q.contiguous(), k.contiguous(), v.contiguous(), int(causal),
                            float(scale), float(beta), int(stable_flag))

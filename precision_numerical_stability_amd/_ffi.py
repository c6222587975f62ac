"""ctypes view of libfa_stable.so: the C ABI declared in include/fa_stable.h, nothing more.

Loading fails loudly (ImportError) when the library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libfa_stable.so")

FA_OK = 0
FA_ERR_NULL = 1
FA_ERR_SHAPE = 2
FA_ERR_HEADDIM = 3
FA_ERR_PARAM = 4
FA_ERR_ALIGN = 5
FA_ERR_HIP = 6
FA_ERR_SCRATCH = 7

FA_FWD_COMPENSATED_SUM = 1

FA_CAUSAL_NONE = 0
FA_CAUSAL_TOP_LEFT = 1
FA_CAUSAL_BOTTOM_RIGHT = 2

FA_ELEM_BF16 = 0
FA_ELEM_F16 = 1

FA_BWD_DELTA = 1
FA_BWD_DKDV = 2
FA_BWD_DQ = 4
FA_BWD_ALL = 7

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float

SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _I, _P]),
    "fa_fwd_ex": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _I, _P]),
    "fa_fwd_stats": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _I, _I, _P]),
    "fa_fwd_qk": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _I, _I, _P]),
    "fa_bwd_qk": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _I, _I, _P]),
    "fa_fwd_elem": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _I, _I, _I, _P]),
    "fa_fwd_diag": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _I, _I, _I, _P]),
    "fa_bwd_elem": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _I, _I, _I, _P]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _I, _P]),
    "fa_bwd_ex": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _I, _I, _P]),
    "fa_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "fa_bwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _I, _P]),
    "fa_bwd_noalloc_max_rows": (ctypes.c_size_t, []),
    "fa_fwd_fp8pv": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _I, _I, _P]),
    "fa_fwd_fp8pv_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "fa_fwd_kv_block": (_I, [_I, _I]),
    "fa_status_str": (ctypes.c_char_p, [_I]),
    "fa_last_hip_error": (_I, []),
}

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once and declare every entry point's signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -m precision_numerical_stability_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def hip_runtimes_mapped() -> list:
    """Distinct libamdhip64 files mapped into this process (there must be exactly one)."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                parts = line.split()
                if len(parts) >= 6 and "libamdhip64" in parts[-1]:
                    paths.add(os.path.realpath(parts[-1]))
    except OSError:
        pass
    return sorted(paths)

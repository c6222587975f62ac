"""C ABI checks that need no GPU: the library loads, exports what include/fa_stable.h declares,
and rejects bad arguments before any HIP call (fake pointers are never dereferenced).

A call whose arguments are all valid gets as far as a kernel launch; with the fake pointers used
here that launch may only happen on a host without a GPU (where it fails with a HIP error), so
every such case sits in a test skipped where a GPU is present."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_stable.h")


def _load_ffi():
    """The ctypes declarations, loaded by path so that the package (which imports torch and loads
    the built library) is not imported by the ABI cases themselves."""
    import importlib.util
    path = os.path.join(ROOT, "precision_numerical_stability_amd", "_ffi.py")
    spec = importlib.util.spec_from_file_location("_fa_ffi_abi_test", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def ffi():
    return _load_ffi()


@pytest.fixture(scope="module")
def lib(ffi):
    # FA_ABI_TEST_LIBRARY selects another build of the same library (the sanitizer test runs
    # these cases against a host build instrumented with AddressSanitizer and UBSan, without torch).
    path = os.environ.get("FA_ABI_TEST_LIBRARY")
    if path is None:
        # As in the package: torch first, so that the library binds to torch's HIP runtime and the
        # binding tests below, which import torch, still see one runtime in this process.
        import torch  # noqa: F401
        path = ffi.LIB_PATH
    return ffi.load_library(path)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib, ffi):
    names = _declared_functions()
    assert set(names) == set(ffi.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for st in range(8):
        s = lib.fa_status_str(st).decode()
        assert s.startswith("FA_")
    assert "unknown" in lib.fa_status_str(99).decode()


def test_workspace_and_block_queries(lib):
    assert lib.fa_bwd_workspace_bytes(1, 32, 8192, 128) == 32 * 8192 * 4
    assert lib.fa_bwd_workspace_bytes(2, 3, 5, 64) == 2 * 3 * 5 * 4
    assert lib.fa_bwd_workspace_bytes(-1, 3, 5, 64) == 0
    assert lib.fa_bwd_workspace_bytes(1, 1, 8, 96) == 0
    for causal in (0, 1):
        assert lib.fa_fwd_kv_block(64, causal) > 0 and lib.fa_fwd_kv_block(128, causal) > 0
        assert lib.fa_fwd_kv_block(80, causal) == 0


P = ctypes.c_void_p(0x7F0000000000)  # 16-byte aligned, never dereferenced
MIS = ctypes.c_void_p(0x7F0000000008)  # 8-byte aligned only


def _fwd(lib, q=P, k=P, v=P, o=P, lse=P, dup=None, ones=None, B=1, H=2, N=128, d=64, causal=0,
         scale=0.125, beta=1.25, flag=1):
    return lib.fa_fwd_ex(q, k, v, o, lse, dup, ones, B, H, N, d, causal, scale, beta, flag, None)


def _bwd(lib, ptrs=None, B=1, H=2, N=128, d=64, causal=0, scale=0.125, beta=1.25, flag=0):
    p = list(ptrs or [P] * 10)
    return lib.fa_bwd(*p, B, H, N, d, causal, scale, beta, flag, None)


def test_forward_validation(lib, ffi):
    assert _fwd(lib, q=None) == ffi.FA_ERR_NULL
    assert _fwd(lib, lse=None) == ffi.FA_ERR_NULL
    assert _fwd(lib, B=-1) == ffi.FA_ERR_SHAPE
    assert _fwd(lib, N=-5) == ffi.FA_ERR_SHAPE
    assert _fwd(lib, B=1 << 20, H=1 << 12) == ffi.FA_ERR_SHAPE
    assert _fwd(lib, N=1 << 30, H=1 << 10) == ffi.FA_ERR_SHAPE
    assert _fwd(lib, N=(1 << 23), d=128, H=1) == ffi.FA_ERR_SHAPE  # one head over 2 GiB
    for d in (0, 32, 96, 256):
        assert _fwd(lib, d=d) == ffi.FA_ERR_HEADDIM
    for scale in (0.0, -1.0, float("nan"), float("inf")):
        assert _fwd(lib, scale=scale) == ffi.FA_ERR_PARAM
    for beta in (0.5, 0.999, float("nan"), float("inf")):
        assert _fwd(lib, beta=beta) == ffi.FA_ERR_PARAM
    for flag in (-1, 3):
        assert _fwd(lib, flag=flag) == ffi.FA_ERR_PARAM
    for causal in (-1, 2):
        assert _fwd(lib, causal=causal) == ffi.FA_ERR_PARAM
    assert _fwd(lib, v=MIS) == ffi.FA_ERR_ALIGN
    assert _fwd(lib, o=MIS) == ffi.FA_ERR_ALIGN
    assert _fwd(lib, lse=ctypes.c_void_p(0x7F0000000002)) == ffi.FA_ERR_ALIGN
    assert _fwd(lib, dup=ctypes.c_void_p(0x7F0000000001)) == ffi.FA_ERR_ALIGN


def test_backward_validation(lib, ffi):
    for i in range(10):
        ptrs = [P] * 10
        ptrs[i] = None
        assert _bwd(lib, ptrs) == ffi.FA_ERR_NULL, i
    for i in (0, 1, 2, 3, 5, 6, 7, 8):  # bf16 tensors need 16-byte alignment
        ptrs = [P] * 10
        ptrs[i] = MIS
        assert _bwd(lib, ptrs) == ffi.FA_ERR_ALIGN, i
    assert _bwd(lib, d=100) == ffi.FA_ERR_HEADDIM
    assert _bwd(lib, scale=-0.1) == ffi.FA_ERR_PARAM
    assert _bwd(lib, flag=7) == ffi.FA_ERR_PARAM
    assert _bwd(lib, H=-2) == ffi.FA_ERR_SHAPE
    for stages in (0, 8, -1):
        assert lib.fa_bwd_ex(*([P] * 10), 1, 2, 128, 64, 0, 0.125, 1.25, 0, stages, None) == ffi.FA_ERR_PARAM
    assert lib.fa_bwd_ex(*([P] * 9), None, 1, 2, 128, 64, 0, 0.125, 1.25, 0, 2, None) == ffi.FA_ERR_NULL


def test_empty_problem_is_a_noop(lib, ffi):
    # no rows: success without touching (here: NULL) pointers and without any HIP call
    assert lib.fa_fwd_ex(None, None, None, None, None, None, None, 0, 4, 128, 64, 0, 0.125, 1.25, 1, None) == 0
    assert lib.fa_fwd(None, None, None, None, None, 3, 4, 0, 128, 1, 0.125, 1.25, 2, None) == 0
    assert _bwd(lib, [None] * 10, B=2, H=0) == ffi.FA_OK
    # parameters are still checked on empty problems
    assert lib.fa_fwd(None, None, None, None, None, 0, 4, 128, 80, 0, 0.125, 1.25, 1, None) == ffi.FA_ERR_HEADDIM


def _gpu_present():
    return os.path.exists("/dev/kfd")


@pytest.mark.skipif(_gpu_present(), reason="needs a host without a GPU (fake pointers would be launched)")
def test_valid_arguments_without_a_device_report_hip_error(lib, ffi):
    assert _fwd(lib) == ffi.FA_ERR_HIP
    assert lib.fa_last_hip_error() == 100  # hipErrorNoDevice
    assert _bwd(lib) == ffi.FA_ERR_HIP


def test_binding_names_match_abi():
    import precision_numerical_stability_amd as fa
    for name in _declared_functions():
        assert callable(getattr(fa, name)), name


def test_single_hip_runtime_mapped():
    import precision_numerical_stability_amd  # noqa: F401
    from precision_numerical_stability_amd import _ffi
    assert len(_ffi.hip_runtimes_mapped()) <= 1


def test_bwd_noalloc_validates_before_any_hip_call(lib, ffi):
    def call(B=1, H=2, N=128, d=64, causal=0, ptrs=None, scale=0.125):
        p = list(ptrs or [P] * 9)
        return lib.fa_bwd_noalloc(*p, B, H, N, d, causal, scale, 1.25, 0, None)
    assert lib.fa_bwd_noalloc_max_rows() == 1 << 21
    assert call(d=80) == ffi.FA_ERR_HEADDIM
    assert call(causal=2) == ffi.FA_ERR_PARAM
    assert call(scale=0.0) == ffi.FA_ERR_PARAM
    assert call(N=-1) == ffi.FA_ERR_SHAPE
    assert call(ptrs=[P] * 8 + [None]) == ffi.FA_ERR_NULL
    assert call(ptrs=[MIS] + [P] * 8) == ffi.FA_ERR_ALIGN
    assert call(B=0) == ffi.FA_OK  # empty: no-op
    # one row beyond the scratch: rejected before any launch (fake pointers stay untouched)
    assert call(B=1, H=1, N=(1 << 21) + 1) == ffi.FA_ERR_SCRATCH
    assert "FA_ERR_SCRATCH" in lib.fa_status_str(ffi.FA_ERR_SCRATCH).decode()


@pytest.mark.skipif(_gpu_present(), reason="needs a host without a GPU (fake pointers would be launched)")
def test_bwd_noalloc_without_a_device_reports_hip_error(lib, ffi):
    assert lib.fa_bwd_noalloc(*([P] * 9), 1, 2, 128, 64, 0, 0.125, 1.25, 0, None) == ffi.FA_ERR_HIP


def test_fwd_diag_validates_and_matches_elem(lib, ffi):
    def call(mshift=P, elem=0, q=P, flags=0):
        return lib.fa_fwd_diag(q, P, P, P, P, None, None, None, None, mshift, 1, 2, 128, 128, 64, 0,
                               0.125, 1.25, 1, flags, elem, None)
    assert call(elem=2) == ffi.FA_ERR_PARAM
    assert call(flags=2) == ffi.FA_ERR_PARAM
    assert call(q=None) == ffi.FA_ERR_NULL
    assert call(mshift=ctypes.c_void_p(0x7F0000000002)) == ffi.FA_ERR_ALIGN
    # shapes and scalars are checked before pointers, as for fa_fwd_elem
    assert lib.fa_fwd_diag(None, P, P, P, P, None, None, None, None, None, 1, 2, 128, 128, 80, 0,
                           0.125, 1.25, 1, 0, 0, None) == ffi.FA_ERR_HEADDIM
    # an empty problem is a no-op whatever the pointers
    assert lib.fa_fwd_diag(None, None, None, None, None, None, None, None, None, None, 0, 2, 128, 128,
                           64, 0, 0.125, 1.25, 1, 0, 0, None) == ffi.FA_OK


def test_fwd_stats_rejects_bad_arguments(lib):
    def call(smin=P, smax=P, flags=0, q=P):
        return lib.fa_fwd_stats(q, P, P, P, P, None, None, smin, smax, 1, 2, 128, 64, 0, 0.125, 1.25,
                                1, flags, None)
    assert call(flags=2) == 4  # FA_ERR_PARAM: unknown flag bit
    assert call(flags=-1) == 4
    assert call(q=None) == 1  # FA_ERR_NULL
    assert call(smin=ctypes.c_void_p(0x7F0000000002)) == 5  # FA_ERR_ALIGN
    assert call(smax=ctypes.c_void_p(0x7F0000000001)) == 5


def _fwd_qk(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Nq=128, Nk=64, d=64, causal=2, flags=0):
    return lib.fa_fwd_qk(q, k, v, o, lse, None, None, None, None, B, H, Nq, Nk, d, causal, 0.125, 1.25,
                         1, flags, None)


def _bwd_qk(lib, ptrs=None, B=1, H=2, Nq=128, Nk=64, d=64, causal=2, stages=7):
    p = list(ptrs or [P] * 10)
    return lib.fa_bwd_qk(*p, B, H, Nq, Nk, d, causal, 0.125, 1.25, 1, stages, None)


def test_qk_entry_points_validate(lib, ffi):
    for causal in (-1, 3):
        assert _fwd_qk(lib, causal=causal) == ffi.FA_ERR_PARAM
        assert _bwd_qk(lib, causal=causal) == ffi.FA_ERR_PARAM
    assert _fwd_qk(lib, Nk=-1) == ffi.FA_ERR_SHAPE and _bwd_qk(lib, Nq=-1) == ffi.FA_ERR_SHAPE
    assert _fwd_qk(lib, Nk=1 << 23, d=128) == ffi.FA_ERR_SHAPE  # one head's keys over 2 GiB
    assert _fwd_qk(lib, flags=4) == ffi.FA_ERR_PARAM
    assert _fwd_qk(lib, k=None) == ffi.FA_ERR_NULL and _fwd_qk(lib, lse=None) == ffi.FA_ERR_NULL
    assert _fwd_qk(lib, v=MIS) == ffi.FA_ERR_ALIGN
    # k and v may be NULL when there are no keys; nothing runs when there are no queries
    assert _fwd_qk(lib, q=None, k=None, v=None, o=None, lse=None, Nq=0) == ffi.FA_OK
    assert _fwd_qk(lib, B=0, q=None) == ffi.FA_OK
    for i in range(10):
        ptrs = [P] * 10
        ptrs[i] = None
        assert _bwd_qk(lib, ptrs) == ffi.FA_ERR_NULL, i
    assert _bwd_qk(lib, [None] * 10, Nq=0, Nk=0) == ffi.FA_OK
    assert _bwd_qk(lib, stages=0) == ffi.FA_ERR_PARAM
    # the square entry points keep accepting only causal 0 or 1
    assert lib.fa_fwd(P, P, P, P, P, 1, 2, 128, 64, 2, 0.125, 1.25, 1, None) == ffi.FA_ERR_PARAM
    assert _bwd(lib, causal=2) == ffi.FA_ERR_PARAM


@pytest.mark.skipif(_gpu_present(), reason="needs a host without a GPU (fake pointers would be launched)")
def test_qk_without_a_device_reports_hip_error(lib, ffi):
    # Nq == 0: the forward is a no-op, the backward still has dK/dV to clear (a launch)
    assert _fwd_qk(lib, Nq=0) == ffi.FA_OK
    assert _bwd_qk(lib, Nq=0) == ffi.FA_ERR_HIP
    assert _fwd_qk(lib, Nk=0, k=None, v=None) == ffi.FA_ERR_HIP


def _fwd_elem(lib, elem, q=P, B=1, H=2, Nq=128, Nk=64, d=64, causal=2):
    return lib.fa_fwd_elem(q, P, P, P, P, None, None, None, None, B, H, Nq, Nk, d, causal, 0.125, 1.25,
                           1, 0, elem, None)


def _bwd_elem(lib, elem, ptrs=None, B=1, H=2, Nq=128, Nk=64, d=64, causal=2, stages=7):
    p = list(ptrs or [P] * 10)
    return lib.fa_bwd_elem(*p, B, H, Nq, Nk, d, causal, 0.125, 1.25, 1, stages, elem, None)


def test_elem_entry_points_validate(lib, ffi):
    for elem in (-1, 2, 7):
        assert _fwd_elem(lib, elem) == ffi.FA_ERR_PARAM
        assert _bwd_elem(lib, elem) == ffi.FA_ERR_PARAM
    for elem in (ffi.FA_ELEM_BF16, ffi.FA_ELEM_F16):
        # the other checks run first and are the same for both element types
        assert _fwd_elem(lib, elem, q=None) == ffi.FA_ERR_NULL
        assert _fwd_elem(lib, elem, d=96) == ffi.FA_ERR_HEADDIM
        assert _fwd_elem(lib, elem, causal=3) == ffi.FA_ERR_PARAM
        assert _bwd_elem(lib, elem, [P] * 9 + [None]) == ffi.FA_ERR_NULL
        assert _bwd_elem(lib, elem, stages=8) == ffi.FA_ERR_PARAM
        assert _fwd_elem(lib, elem, B=0, q=None) == ffi.FA_OK
        assert _bwd_elem(lib, elem, [None] * 10, Nq=0, Nk=0) == ffi.FA_OK
    # the element type is checked even where nothing would run
    assert _fwd_elem(lib, 2, B=0, q=None) == ffi.FA_ERR_PARAM


@pytest.mark.skipif(_gpu_present(), reason="needs a host without a GPU (fake pointers would be launched)")
def test_elem_without_a_device_reports_hip_error(lib, ffi):
    for elem in (ffi.FA_ELEM_BF16, ffi.FA_ELEM_F16):
        assert _fwd_elem(lib, elem) == ffi.FA_ERR_HIP
        assert _bwd_elem(lib, elem) == ffi.FA_ERR_HIP


def test_binding_rejects_mixed_or_unsupported_dtypes():
    import torch
    import precision_numerical_stability_amd as fa
    with pytest.raises(ValueError):
        fa._elem(torch.zeros(1, dtype=torch.float32), "q")
    assert fa._elem(torch.zeros(1, dtype=torch.float16), "q") == fa.FA_ELEM_F16
    assert fa._elem(torch.zeros(1, dtype=torch.bfloat16), "q") == fa.FA_ELEM_BF16


def test_fp8pv_entry_point_validates(lib, ffi):
    def call(ws=P, q=P, B=1, H=2, Nq=128, Nk=300, d=64, causal=1, flag=1, flags=0):
        return lib.fa_fwd_fp8pv(q, P, P, P, P, None, None, None, None, ws, B, H, Nq, Nk, d, causal,
                                0.125, 1.25, flag, flags, None)
    assert call(ws=None) == ffi.FA_ERR_NULL
    assert call(ws=MIS) == ffi.FA_ERR_ALIGN
    assert call(q=None) == ffi.FA_ERR_NULL
    assert call(d=96) == ffi.FA_ERR_HEADDIM and call(flag=3) == ffi.FA_ERR_PARAM
    assert call(causal=3) == ffi.FA_ERR_PARAM and call(flags=2) == ffi.FA_ERR_PARAM
    assert call(B=0, q=None, ws=None) == ffi.FA_OK
    assert lib.fa_fwd_fp8pv_workspace_bytes(1, 2, 300, 64) == 2 * 3 * (64 * 128 + 4)
    assert lib.fa_fwd_fp8pv_workspace_bytes(1, 32, 8192, 128) == 32 * 64 * (128 * 128 + 4)
    assert lib.fa_fwd_fp8pv_workspace_bytes(1, 1, 0, 128) == 0
    assert lib.fa_fwd_fp8pv_workspace_bytes(1, 1, 8, 80) == 0


@pytest.mark.skipif(_gpu_present(), reason="needs a host without a GPU (fake pointers would be launched)")
def test_fp8pv_without_keys_needs_no_workspace_without_a_device(lib, ffi):
    # No keys: the NULL workspace is accepted and the call goes on to launch (which fails here).
    assert lib.fa_fwd_fp8pv(P, P, P, P, P, None, None, None, None, None, 1, 2, 128, 0, 64, 1, 0.125,
                            1.25, 1, 0, None) == ffi.FA_ERR_HIP

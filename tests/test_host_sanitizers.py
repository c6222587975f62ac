"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The C ABI's host side (fa_api.cpp: validation, dispatch, the no-allocation scratch lookup) is
rebuilt with the sanitizers on its host pass only, linked with the library's kernel objects into a
separate shared library, and the ABI validation cases of test_abi.py run against it in a
subprocess that preloads the sanitizer runtime.  Any report aborts that subprocess.  A second
test plants an out-of-bounds read and a signed overflow in a throwaway library built the same way,
to show that this harness does report them.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "precision_numerical_stability_amd", "csrc")
OBJ = os.path.join(ROOT, "precision_numerical_stability_amd", "_lib", "obj")
KERNEL_OBJS = ("fa_fwd_bf16.o", "fa_fwd_f16.o", "fa_fwd_fp8pv.o", "fa_bwd_bf16.o", "fa_bwd_f16.o")

# Sanitizers on the host pass only: each -fsanitize= goes behind -Xarch_host, so no device code
# is instrumented.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return path if os.path.exists(path) else None


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _need_toolchain():
    if _hipcc() is None or _asan_runtime() is None:
        pytest.skip("hipcc or the clang sanitizer runtime is not installed")
    missing = [o for o in KERNEL_OBJS if not os.path.exists(os.path.join(OBJ, o))]
    if missing:
        pytest.skip(f"library objects not built yet: {missing}")


def _compile(src, obj):
    cmd = [_hipcc(), "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-3000:]


def _link(objs, out):
    res = subprocess.run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-3000:]


def _env(extra=None):
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra or {})
    return env


def test_abi_cases_under_asan_and_ubsan(tmp_path):
    _need_toolchain()
    obj = str(tmp_path / "fa_api_san.o")
    _compile(os.path.join(CSRC, "fa_api.cpp"), obj)
    so = str(tmp_path / "libfa_stable_san.so")
    _link([obj, *(os.path.join(OBJ, o) for o in KERNEL_OBJS)], so)
    nm = shutil.which("nm")
    if nm:
        syms = subprocess.run([nm, "-D", so], capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms, "the host code is not instrumented"
    res = subprocess.run(
        [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-p",
         "no:cacheprovider", "-k", "not binding and not single_hip_runtime"],
        cwd=str(tmp_path), env=_env({"FA_ABI_TEST_LIBRARY": so}), capture_output=True, text=True,
        timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out


PLANTED = r"""
#include <climits>
#include <hip/hip_runtime.h>
extern "C" int planted_oob(int i) {
  int* a = new int[4]();
  int r = a[i];
  delete[] a;
  return r;
}
extern "C" int planted_overflow(int x) { return x + INT_MAX; }
"""


@pytest.mark.parametrize("fn,arg,report", [("planted_oob", 4, "heap-buffer-overflow"),
                                           ("planted_overflow", 1, "signed integer overflow")])
def test_the_harness_reports_planted_errors(tmp_path, fn, arg, report):
    _need_toolchain()
    src = tmp_path / "planted.cpp"
    src.write_text(PLANTED)
    obj = str(tmp_path / "planted.o")
    _compile(str(src), obj)
    so = str(tmp_path / "libplanted.so")
    _link([obj], so)
    code = f"import ctypes; ctypes.CDLL({so!r}).{fn}({arg}); print('no report')"
    res = subprocess.run([sys.executable, "-c", code], env=_env(), capture_output=True, text=True,
                         timeout=120)
    out = res.stdout + res.stderr
    assert res.returncode != 0 and report in out, out[-3000:]

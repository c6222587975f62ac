"""Build the HIP library for gfx950: hipcc compiles each translation unit, then links one shared
library, ``_lib/libfa_stable.so``, next to this file.  Run as ``python
precision_numerical_stability_amd/build.py`` (``--jobs N`` to limit parallel compiles); it does not
import the package, which would load the library being rebuilt."""
from __future__ import annotations

import argparse
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "_lib")
LIBNAME = "libfa_stable.so"
# (source, object name, extra defines).  The kernel files are compiled once per element type:
# FA_ELEM=0 instantiates the bf16 kernels, FA_ELEM=1 the fp16 ones, FA_ELEM=2 (forward only)
# the bf16 forward with an FP8 P^ V product and its V quantisation kernel.
UNITS = (
    ("fa_fwd.hip", "fa_fwd_bf16", ("-DFA_ELEM=0",)),
    ("fa_fwd.hip", "fa_fwd_f16", ("-DFA_ELEM=1",)),
    ("fa_fwd.hip", "fa_fwd_fp8pv", ("-DFA_ELEM=2",)),
    ("fa_bwd.hip", "fa_bwd_bf16", ("-DFA_ELEM=0",)),
    ("fa_bwd.hip", "fa_bwd_f16", ("-DFA_ELEM=1",)),
    ("fa_api.cpp", "fa_api", ()),
)
SOURCES = tuple(sorted({u[0] for u in UNITS}))
ARCH = "gfx950"

# -packed-fp32-ops keeps the compiler from forming packed fp32 VALU instructions.
COMMON_FLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build the library")
    return path


def _compile(src: str, obj: str, extra) -> None:
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {src}")


def build(jobs: int = 3, extra=()) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, name + ".o") for _, name, _ in UNITS]
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        futs = [ex.submit(_compile, src, o, [*defs, *extra]) for (src, _, defs), o in zip(UNITS, objs)]
        for f in futs:
            f.result()
    out = os.path.join(LIBDIR, LIBNAME)
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking libfa_stable.so failed")
    _check_no_undefined_stubs(tmp)
    os.replace(tmp, out)
    return out


def _check_no_undefined_stubs(lib: str) -> None:
    """Fail the build if the library references a kernel launch stub it does not define."""
    nm = shutil.which("nm")
    if nm is None:
        return
    res = subprocess.run([nm, "-D", "--undefined-only", lib], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in res.stdout.splitlines() if "__device_stub__" in ln]
    if missing:
        raise RuntimeError(f"{len(missing)} kernel launch stubs are undefined in {lib}, e.g. {missing[0]}")


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=3)
    args = ap.parse_args()
    print(build(args.jobs))

"""Build libbatq.so (all HIP sources, gfx950) in-tree with hipcc, and
libbatq_vendor.so (the hipBLASLt comparison GEMM of include/batq_vendor.h).

Each source compiles to its own object in parallel (the GEMM files fully
unroll their stage loops and dominate the time), then one link makes the
shared library.  Objects go to a scratch folder beside the package and are
rebuilt on every call.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libbatq.so")
# hipBLASLt's MXFP4 GEMM behind include/batq_vendor.h: a comparison for the
# benchmark, linked on its own so that libbatq.so does not depend on hipBLASLt
VENDOR_LIB = os.path.join(PKG, "libbatq_vendor.so")
VENDOR_SRC = os.path.join(PKG, "vendor", "hipblaslt_mxfp4.cpp")
OBJ_DIR = os.path.join(PKG, "_build")

COMPILE_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    # packed FP32 math stays off (the compiler would otherwise emit v_pk_* ops)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # the GEMM kernels fully unroll their stage loops for common K (exact wait counts)
    "-mllvm", "-pragma-unroll-threshold=1000000",
    # leading scalar kernel arguments arrive in SGPRs at wave launch, so a
    # latency-bound kernel (the fused decode step) issues its first loads
    # without waiting for a scalar load of its arguments; aggregate arguments
    # are unaffected, and firmware without preloading runs the loading prologue
    # the compiler emits
    "-mllvm", "-amdgpu-kernarg-preload-count=8",
]
LINK_FLAGS = ["--offload-arch=gfx950", "-shared", "-fPIC"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _filter(stderr: str) -> str:
    return "\n".join(ln for ln in stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip())


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMPILE_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({res.returncode}):\n{_filter(res.stderr)}")
    if verbose and _filter(res.stderr):
        print(_filter(res.stderr), file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *LINK_FLAGS, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc link failed ({res.returncode}):\n{_filter(res.stderr)}")
    os.replace(tmp, LIB)
    build_vendor(verbose)
    return LIB


def build_vendor(verbose: bool = False) -> str:
    tmp = VENDOR_LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-shared", "-I", os.path.join(ROOT, "include"),
           VENDOR_SRC, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lhipblaslt", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(VENDOR_SRC)} ({res.returncode}):\n{_filter(res.stderr)}")
    os.replace(tmp, VENDOR_LIB)
    return VENDOR_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libcnhwc.so (the HIP kernels + C ABI) in-tree with hipcc for gfx950.

Every source is compiled on every call (the build check must really compile),
in parallel, then linked into convolution_nhwc_conv2d_amd/libcnhwc.so.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcnhwc.so")
OBJDIR = os.path.join(PKG, "_build")
SOURCES = ["select.cpp", "api.cpp", "gemm.hip", "gemm_lds.hip", "wino_gemm.hip", "winograd.hip", "winograd_h.hip", "unfold.hip", "noalloc.hip", "gemm_patch.hip"]
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          # packed fp32 VALU forms stay off (only ordinary fp32 instructions are emitted)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.exists(c) or c == "hipcc":
            return c


def _compile(src, verbose):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc()] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    # the Winograd matrices header is generated from exact rationals
    subprocess.run([sys.executable, os.path.join(CSRC, "gen_winograd.py")], check=True,
                   capture_output=not verbose)
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

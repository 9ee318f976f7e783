"""Build libtl.so (gfx950 HIP kernels + host engine) in-tree with hipcc.

build(sanitize=True) builds libtl_asan.so instead: the host engine (engine.cpp:
argument checks, staging, the KV arena allocator, descriptors, graph capture) is
compiled by g++ under AddressSanitizer and UndefinedBehaviorSanitizer and linked
with the unchanged HIP objects.  g++'s runtimes are used rather than the HIP
compiler's, whose AddressSanitizer also intercepts the HSA runtime's device
allocations (that is GPU-side sanitizing, which needs xnack).  The library is
loaded through TL_LIBRARY with sanitizer_runtimes() preloaded, for test runs.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtl.so")
OBJ_ASAN = os.path.join(HERE, "_build_asan")
LIB_ASAN = os.path.join(HERE, "libtl_asan.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
GXX = os.environ.get("CXX", "g++")
SANITIZE = ["-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer", "-g"]


def sanitizer_runtimes() -> list:
    """g++'s shared AddressSanitizer and UndefinedBehaviorSanitizer runtimes (to be
    preloaded, in this order), or [] when they are not installed."""
    out = []
    for name in ("libasan.so", "libubsan.so"):
        r = subprocess.run([GXX, "-print-file-name=" + name], capture_output=True, text=True)
        path = r.stdout.strip()
        if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
            return []
        out.append(path)
    return out


def _compile(src: str, sanitize: bool = False) -> str:
    if src.endswith(".hip"):
        # the sanitized build links the ordinary HIP objects
        obj = os.path.join(OBJ, os.path.basename(src) + ".o")
        if sanitize and os.path.exists(obj) and os.path.getmtime(obj) >= _newest_source():
            return obj
        cmd = [HIPCC, *COMMON, *DEVICE, "-c", src, "-o", obj]
    elif sanitize:
        obj = os.path.join(OBJ_ASAN, os.path.basename(src) + ".o")
        cmd = [GXX, *COMMON, *SANITIZE, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c", src, "-o", obj]
    else:
        obj = os.path.join(OBJ, os.path.basename(src) + ".o")
        cmd = [HIPCC, *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def _newest_source() -> float:
    return max(os.path.getmtime(f) for f in glob.glob(os.path.join(CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*")))


def build(verbose: bool = False, sanitize: bool = False) -> str:
    lib = LIB_ASAN if sanitize else LIB
    os.makedirs(OBJ, exist_ok=True)
    os.makedirs(OBJ_ASAN, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), srcs))
    tmp = lib + ".tmp"
    # the sanitized library leaves the runtimes' symbols to the preloaded runtimes
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv)
    sys.exit(0)

"""Build the gfx950 C-ABI library in place:
diffusion_drafted_verification_amd/liborthrus_gfx950.so.

    python -m diffusion_drafted_verification_amd.build

Each .hip source is compiled separately for gfx950 (hipcc cross-compiles
without a GPU) and linked into one shared library whose only interface is
include/orthrus.h.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "liborthrus_gfx950.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["block_attn.hip", "greedy_accept.hip", "kv_append.hip", "sample_accept.hip", "lm_head.hip", "prefill.hip"]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc")


def compile_flags():
    return ["-std=c++17", "-O3", f"--offload-arch={ARCH}", "-fPIC", "-I", INCLUDE, "-I", CSRC,
            "-Wall", "-Wno-unused-function",
            # keep fp32 arithmetic off the packed-fp32 VALU forms
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-munsafe-fp-atomics"]


def _compile(src):
    out = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [hipcc(), *compile_flags(), "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    return out, errs


def build(verbose=True):
    cc = hipcc()
    if not cc:
        raise RuntimeError("hipcc not found (ROCm is required to build the gfx950 library)")
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    for (obj, errs), src in zip(results, SOURCES):
        if errs and verbose:
            print(f"[{src}]\n{errs}", file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build()

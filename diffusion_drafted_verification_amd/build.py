"""Build the gfx950 C-ABI library in place:
diffusion_drafted_verification_amd/liborthrus_gfx950.so.

    python -m diffusion_drafted_verification_amd.build
    python -m diffusion_drafted_verification_amd.build --sanitize   (the same
        library with AddressSanitizer + UBSan on its host code, under
        _build/sanitize, for the CPU tests of the argument validation)

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


SANITIZE_DIR = os.path.join(BUILD, "sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, LIB_NAME)


def sanitize_flags():
    """AddressSanitizer and UndefinedBehaviorSanitizer on the host code only
    (the C-ABI validation and launch set-up); the gfx950 device code is built
    as usual, without sanitizers."""
    return [*compile_flags(), "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]


def asan_runtime():
    """Path of the compiler's AddressSanitizer runtime (to preload into a
    Python process that loads the sanitized library), or None."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    base = os.path.join(rocm, "llvm", "lib", "clang")
    if not os.path.isdir(base):
        return None
    for v in sorted(os.listdir(base), reverse=True):
        p = os.path.join(base, v, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def build_sanitized(verbose=True, force=False):
    """Build the sanitized library (skipped when it is newer than every source
    and header it is built from, unless force)."""
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]
    deps.append(os.path.abspath(__file__))
    if not force and os.path.exists(SANITIZE_LIB) and \
            os.path.getmtime(SANITIZE_LIB) > max(os.path.getmtime(p) for p in deps):
        return SANITIZE_LIB

    def one(src):
        out = os.path.join(SANITIZE_DIR, src.replace(".hip", ".o"))
        r = subprocess.run([hipcc(), *sanitize_flags(), "-c", os.path.join(CSRC, src), "-o", out],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (sanitized build) failed on {src}:\n{r.stderr}")
        return out

    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address,undefined",
                        "-o", SANITIZE_LIB, *objs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (sanitized build) failed:\n{r.stderr}")
    if verbose:
        print(f"built {SANITIZE_LIB}")
    return SANITIZE_LIB


# Per-source flags.  block_attn.hip: preload the leading scalar arguments of
# the streaming attention and combine kernels (context lengths, page table,
# partial buffers, decomposition) into SGPRs at wave start, so their first
# loads do not wait for a kernel-argument load (B1 decode call 17.9 -> 17.4
# us with the attention kernel's six).
SOURCE_FLAGS = {"block_attn.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=10"],
                "greedy_accept.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=4"],
                "sample_accept.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=7"]}


def _compile(src):
    out = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [hipcc(), *compile_flags(), *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", out]
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
    if "--sanitize" in sys.argv[1:]:
        build_sanitized(force=True)
    else:
        build()

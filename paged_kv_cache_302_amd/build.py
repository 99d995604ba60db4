"""Build libpa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m paged_kv_cache_302_amd.build [--debug]

The library is written next to this file so that it travels with the source
tree; the Python binding loads it from there.  `sanitize=True` builds a copy
whose host code (the C ABI's argument checks, the block manager) carries
AddressSanitizer and UndefinedBehaviorSanitizer, for CPU tests only: the
device code is built as usual, and the sanitizer runtime must be preloaded
(see ASAN_RUNTIME).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa.so")
SOURCES = ["pa_api.hip", "pa_decode.hip", "pa_prefill.hip", "pa_reduce.hip", "pa_cache.hip",
           "pa_noalloc.hip", "pa_blocks.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


# host-only sanitizer flags: each one applies to the host pass only
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-g"]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime a sanitized build needs preloaded."""
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang's AddressSanitizer runtime was not found under /opt/rocm/llvm")
    return found[-1]


def command(out: str = LIB, debug: bool = False, sanitize: bool = False) -> list:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-std=c++17", "-shared", "-fPIC",
           "-O1" if debug or sanitize else "-O3",
           # no packed-fp32 (v_pk_*_f32) code generation
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # MFMA accumulators in ordinary VGPRs: the online-softmax rescale
           # multiplies them every block, which AGPRs would force through copies
           "-mllvm", "-amdgpu-mfma-vgpr-form=true",
           "-fvisibility=hidden", "-I", INCLUDE, "-I", CSRC,
           "-Wno-unused-command-line-argument"]
    if sanitize:
        cmd += SANITIZE_FLAGS
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    cmd += ["-o", out]
    return cmd


def build(out: str = LIB, debug: bool = False, verbose: bool = True, sanitize: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = command(tmp, debug, sanitize)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(debug="--debug" in sys.argv)

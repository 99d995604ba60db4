"""Build libpa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m paged_kv_cache_302_amd.build [--debug]

The library is written next to this file so that it travels with the source
tree; the Python binding loads it from there.
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


def command(out: str = LIB, debug: bool = False) -> list:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-std=c++17", "-shared", "-fPIC",
           "-O1" if debug else "-O3",
           # no packed-fp32 (v_pk_*_f32) code generation
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # MFMA accumulators in ordinary VGPRs: the online-softmax rescale
           # multiplies them every block, which AGPRs would force through copies
           "-mllvm", "-amdgpu-mfma-vgpr-form=true",
           "-fvisibility=hidden", "-I", INCLUDE, "-I", CSRC,
           "-Wno-unused-command-line-argument"]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    cmd += ["-o", out]
    return cmd


def build(out: str = LIB, debug: bool = False, verbose: bool = True) -> str:
    tmp = out + ".tmp"
    cmd = command(tmp, debug)
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

"""Build the HIP library (libpaged_attn.so) in-tree for gfx950.

Usage: python -m paged_attention_long_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpaged_attn.so")
ARCH = "gfx950"

SOURCES = ["paged_attn.cpp", "pa_decode_valu.hip", "pa_tile_attn.hip", "pa_merge.hip", "pa_gather.hip"]

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
    # Packed FP32 VALU instructions are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    # MFMA accumulators in ordinary VGPRs: no copies between the AGPR and VGPR
    # files around the softmax rescale.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = True, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}", "-o", tmp, *srcs]
    t0 = time.time()
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    # a library with an unresolved symbol must fail the build, not the first caller
    import ctypes

    ctypes.CDLL(os.path.abspath(tmp))
    os.replace(tmp, LIB)
    if verbose:
        warn = [l for l in res.stderr.splitlines() if "warning" in l and "packed-fp32-ops" not in l]
        for l in warn[:20]:
            print(l)
        print(f"built {LIB} in {time.time() - t0:.1f}s")
    return LIB


if __name__ == "__main__":
    build()

"""Build libverify.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m bit_block_scaled_vq_amd.build   (or call build()).
The library lands in bit_block_scaled_vq_amd/lib/libverify.so.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libverify.so")
SOURCES = [os.path.join(CSRC, "libverify.cpp"), os.path.join(CSRC, "vq_kernels.hip"),
           os.path.join(CSRC, "vq_sample.hip"), os.path.join(CSRC, "vq_gdn.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Code generation flags (they decide the kernels' machine code together with
# the sources, so measurements stored with a digest of the sources hash these
# too).
CODEGEN_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the M <= 8 NVFP4 path reads every MFMA
    # result with VALU FMAs, and accumulation registers would add four
    # v_accvgpr_read per MFMA and serialise the MFMAs on one register quad
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # kernel arguments listed first are preloaded into SGPRs at wave launch
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    # the scheduler that favours instruction-level parallelism interleaves
    # the decode, the MFMAs and the next loads better at one wave per SIMD:
    # bitwise the same results, M = 8 pass 4.125 -> 4.105 ms over ten
    # interleaved rounds, the 4-lane pass 5.94 -> 5.82 ms
    "-mllvm", "-amdgpu-sched-strategy=max-ilp",
    "-Wall", "-Wno-unused-command-line-argument",
]
FLAGS = CODEGEN_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = True) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)

"""Build libmsa.so (all HIP kernels + the C ABI) in-tree for gfx950 with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmsa.so")

SOURCES = ["msa_api.hip", "index_scores.hip", "block_topk.hip", "attn_gather.hip",
           "attn_tile.hip", "index_kl.hip", "decode_attn.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Packed fp32 VALU ops stay off: the compiler must not form v_pk_* fp32 math.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Inputs are finite (NaN/Inf inputs are undefined behaviour of the ABI), so the
    # compiler need not quiet MFMA results before every max (IEEE-mode canonicalising
    # v_max_f32 x, x would otherwise double the max-pooling VALU work).
    "-fno-honor-nans",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MSA library needs ROCm's hipcc to build")


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source into libmsa.so next to this file and return its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libmsa.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))

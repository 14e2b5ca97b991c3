"""Build the HIP library libsv.so for gfx950, in place, next to this file.

python -m lossless_draft_verification_sv_amd.build   (or __graft_entry__.build())
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", n) for n in ("sv_kernels.hip", "sv_tags.hip", "sv_probe.hip",
                                                "sv_schedule.hip", "sv_markov.hip",
                                                "sv_markov_topk.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsv.so")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # all floating-point contraction in the kernels is written out explicitly
    "-ffp-contract=off",
    # no packed fp32 instructions (v_pk_*_f32) in any generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsv.so)")


def build(verbose: bool = False) -> str:
    """Compile libsv.so (always recompiles). Returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-o", tmp, *SRCS]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

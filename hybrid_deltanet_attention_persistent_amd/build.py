"""Build the HIP library (libmk.so) in-tree for gfx950 with hipcc.

Usage: python -m hybrid_deltanet_attention_persistent_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmk.so")
SOURCES = ["mk_api.cpp", "mk_forward.hip", "mk_verify.hip", "mk_prefill.hip"]

# -ffp-contract=off: every fused multiply-add in the kernels is an explicit fmaf, so the
# arithmetic (and the bit-identity of decode and verify) is fixed by the source.
# -packed-fp32-ops off: no packed FP32 instructions are generated.
FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile libmk.so from csrc/ (always recompiles).  Returns the library path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + FLAGS + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stderr[-8000:])
    if verbose and res.stderr.strip():
        sys.stderr.write("\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

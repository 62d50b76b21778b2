"""Build libnormgemm.so (HIP, gfx950) in place, next to this file.

    python -m normalization_gemm_amd.build

The library is one translation unit (csrc/ng_api.hip) compiled by hipcc for
gfx950 only.  The output is written to a temporary name and renamed, so a
process that has the old library loaded is not disturbed.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libnormgemm.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

HIPCC_FLAGS = [
    "-O3",
    "--offload-arch=gfx950",
    "-std=c++17",
    "-shared",
    "-fPIC",
    # Keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def build(verbose: bool = False) -> str:
    """Compile the library; return its path.  Raises on compiler failure."""
    src = os.path.join(CSRC, "ng_api.hip")
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.unlink(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, "\n".join(msgs)))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)

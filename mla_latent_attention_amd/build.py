"""Build step: compile the HIP sources under csrc/ into the in-tree libmla.so.

hipcc cross-compiles for gfx950 without a GPU present.  Packed-fp32 VALU
instructions are disabled for the device code (-packed-fp32-ops); the host
pass warns that it does not know that feature, which is harmless.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla.so")
SOURCES = ["mla_decode.hip", "mla_decode_groups.hip", "mla_surround.hip", "mla_api.hip"]
ARCH = "gfx950"

FLAGS = [
    "-O3",
    f"--offload-arch={ARCH}",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build_library(verbose: bool = False) -> str:
    """Compile libmla.so (always recompiles) and return its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))

"""Build step: compile the HIP sources under csrc/ into the in-tree libmla.so,
and the same sources with MLA_DEBUG_CHECKS defined into libmla_debug.so (every
decode entry point first checks its index arguments on the device and
synchronises; see mla_check_inputs in include/mla.h).

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
LIB_DEBUG = os.path.join(HERE, "libmla_debug.so")
SOURCES = ["mla_decode.hip", "mla_decode_groups.hip", "mla_surround.hip", "mla_check.hip",
           "mla_api.hip"]
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
    """Compile libmla.so and libmla_debug.so (always recompiles; the two builds
    run side by side) and return the path of libmla.so."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    jobs = []
    for out, extra in ((LIB, []), (LIB_DEBUG, ["-DMLA_DEBUG_CHECKS"])):
        cmd = [hipcc(), *FLAGS, *extra, *srcs, "-o", out + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                           text=True)))
    noise = "is not a recognized feature for this target"
    failed = []
    for out, proc in jobs:
        _, stderr = proc.communicate()
        err = "\n".join(l for l in stderr.splitlines() if noise not in l)
        if proc.returncode != 0:
            failed.append(f"{os.path.basename(out)}: hipcc failed ({proc.returncode}):\n{err}")
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    if failed:
        raise RuntimeError("\n".join(failed))
    for out, _ in jobs:
        os.replace(out + ".tmp", out)
    return LIB


# The plain-C caller of the C ABI that a GPU test runs (host code only: gcc,
# C11, linked against libmla.so and the HIP runtime, found through rpath).
ROOT = os.path.dirname(HERE)
C_DRIVER_SRC = os.path.join(ROOT, "tests", "native", "c_abi_decode.c")
C_DRIVER = os.path.splitext(C_DRIVER_SRC)[0]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_driver(verbose: bool = False) -> str | None:
    """Compile tests/native/c_abi_decode.c against the built libmla.so (None
    when the tests are not present)."""
    if not os.path.exists(C_DRIVER_SRC):
        return None
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", C_DRIVER_SRC,
           "-o", C_DRIVER + ".tmp", f"-L{HERE}", "-lmla", f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../mla_latent_attention_amd", f"-Wl,-rpath,{ROCM}/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(C_DRIVER + ".tmp", C_DRIVER)
    return C_DRIVER


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_c_driver(verbose=True))

"""Build ``libmla_decode.so`` (gfx950) in-tree with hipcc.

The library links the HIP runtime by its soname ``libamdhip64.so.7``.  Loaded
after ``import torch`` it binds to the runtime torch already loaded (same
soname), so the process holds a single HIP runtime and torch's streams are
valid handles for it.

Usage: ``python -m paged_mla_decode_03_amd.build`` (or ``build()`` from Python).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libmla_decode.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["mla_api.hip", "mla_sched.hip", "mla_decode.hip", "mla_decode_wide.hip", "mla_combine.hip",
           "mla_append.hip", "mla_absorb.hip", "mla_check.hip",
           "mla_outproj.hip", "mla_pages.hip",
           "mla_stream.hip"]
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the generated code; -O3 would
# otherwise form them from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain is required to build the library)")


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source for gfx950 and link the shared library."""
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-shared",
           "-munsafe-fp-atomics", "-I", os.path.join(ROOT, "include"), *DEVICE_FLAGS, *extra_flags,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB_PATH + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-8000:]}")
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

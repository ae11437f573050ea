"""Builds libflashblock.so in-tree with hipcc for gfx950.

    python -m cached_attention_amd.build [-v]

The library links the HIP runtime by soname (libamdhip64.so.7); loaded into a
process that has already imported torch it binds to the runtime torch loaded,
so torch's streams are valid handles for it.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libflashblock.so")
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "fb_api.cpp"), os.path.join(CSRC, "fb_kernels.hip")]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # packed fp32 VALU ops stay off in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compiles every source into cached_attention_amd/libflashblock.so; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}", "-shared",
           "-o", tmp, *SOURCES, "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

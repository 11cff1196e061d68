"""Build the HIP library ``libonline_softmax.so`` for gfx950 with hipcc.

``python online_normalizer_amd/build.py`` compiles in place (run it as a
script: importing it through the package would load the library first).  Packed fp32 VALU
instructions are disabled for all device code (``-packed-fp32-ops``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "os_abi.hip")]
DEPENDS = SOURCES + [os.path.join(HERE, "csrc", f) for f in ("os_device.hpp", "os_kernels.hpp", "os_attention.hpp")] + [
    os.path.join(ROOT, "include", "online_softmax.h")]
LIB = os.path.join(HERE, "libonline_softmax.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(out: str = LIB, extra_flags: list[str] | None = None, verbose: bool = False) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), *SOURCES, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, extra_flags=sys.argv[1:]))

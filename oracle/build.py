"""Compile ``oracle.c`` into ``liboracle.so`` with the host C compiler.

Flags keep IEEE double semantics: no fast-math, no contraction into FMA.
``python -m oracle.build`` builds the default library in place.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_SRC = os.path.join(HERE, "oracle.c")
DEFAULT_LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(src: str = DEFAULT_SRC, out: str = DEFAULT_LIB, cc: str = "gcc",
          werror: bool = True) -> str:
    cmd = [cc, *CFLAGS, *(["-Werror"] if werror else []), src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:]))

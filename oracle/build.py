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
# AddressSanitizer + UndefinedBehaviorSanitizer for a checked CPU build (the
# process that loads it must preload libasan); any report aborts.
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g"]
# Set to "1" to build every oracle library with SANITIZE_FLAGS.
SANITIZE_ENV = "ONORM_ORACLE_SANITIZE"


def sanitizing() -> bool:
    return os.environ.get(SANITIZE_ENV) == "1"


def build(src: str = DEFAULT_SRC, out: str = DEFAULT_LIB, cc: str = "gcc",
          werror: bool = True, sanitize: bool | None = None) -> str:
    if sanitize is None:
        sanitize = sanitizing()
    cmd = [cc, *CFLAGS, *(SANITIZE_FLAGS if sanitize else []), *(["-Werror"] if werror else []), src,
           "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:]))

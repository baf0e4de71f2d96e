"""Build the plain C oracle into ``oracle/liboracle.so`` with gcc (test infrastructure only).

Flags keep IEEE semantics: no fast-math, no FMA contraction, round-to-nearest default.
OpenMP only splits independent output rows of the GEMMs.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "w8a8_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
          "-frounding-math", "-fopenmp", "-Wall", "-Wextra"]


# Address and undefined-behaviour sanitizers, for the sanitized test build (build(path, SANITIZE)).
SANITIZE = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def build(verbose: bool = False, path: str | None = None, extra=()) -> str:
    """Compile the oracle into path (default LIB_PATH) with CFLAGS plus extra."""
    out = LIB_PATH if path is None else path
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", *CFLAGS, *extra, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

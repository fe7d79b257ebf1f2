"""Compile the oracle's C sources into ``oracle/liboracle.so`` (gcc, OpenMP):
the oracle itself (``adaln_oracle.c``) and the row-by-row comparison the
parity tests use (``check_rows.c``, which calls the oracle).

Test infrastructure only; see ``adaln_oracle.c``."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "adaln_oracle.c"),
        os.path.join(HERE, "check_rows.c")]
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Build the oracle library and return its path (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", *SRCS, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

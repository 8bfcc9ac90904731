"""Builds liboracle.so, the fp64 CPU oracle (test infrastructure only).

The product path never loads this library. The target is generic x86-64-v2
so a library built on one host also runs on another.
"""
from __future__ import annotations

import subprocess
import sys
from pathlib import Path

HERE = Path(__file__).resolve().parent
SRC = HERE / "kda_oracle.c"
LIB = HERE / "liboracle.so"


def build(verbose: bool = False) -> Path:
    cmd = ["gcc", "-O3", "-march=x86-64-v2", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", str(LIB) + ".tmp", str(SRC), "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    Path(str(LIB) + ".tmp").replace(LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

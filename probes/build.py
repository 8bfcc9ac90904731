"""Builds libkda_probes.so from ceilings.hip with hipcc, gfx950 only, in-tree.

    python -m probes.build

Measurement probes for bench.py; the operator's library does not include them.
"""
from __future__ import annotations

import subprocess
import sys
from pathlib import Path

HERE = Path(__file__).resolve().parent
SRC = HERE / "ceilings.hip"
LIB = HERE / "libkda_probes.so"


def build(verbose: bool = False) -> Path:
    from gated_delta_rule_50_amd import build as kbuild
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [kbuild.hipcc(), "-x", "hip", *kbuild._flags(), "-shared", "-o", str(tmp), str(SRC)]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for ceilings.hip:\n" + res.stdout + res.stderr)
    tmp.replace(LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Builds libkda.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m gated_delta_rule_50_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, and linked into one shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libkda.so"
BUILD = ROOT / "_build"
SOURCES = ["kda_api.cpp", "kda_prefill.hip", "kda_recurrent.hip", "kda_epilogue.hip",
           "kda_check.hip", "kda_noalloc.hip"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = Path(rocm) / "bin" / "hipcc"
    return str(exe) if exe.exists() else (shutil.which("hipcc") or "hipcc")


def _flags():
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}", "-Wall",
            # keep MFMA accumulators in VGPRs (no AGPR copies around VALU use)
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            *os.environ.get("KDA_EXTRA_FLAGS", "").split()]


def _compile(src, verbose: bool) -> Path:
    path = Path(src) if os.path.isabs(str(src)) else CSRC / src
    out = BUILD / (path.name + ".o")
    cmd = [hipcc(), *_flags(), "-c", str(path), "-o", str(out)]
    if path.suffix == ".hip":
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)
    return out


def _link(objs, lib: Path, verbose: bool) -> None:
    tmp = lib.with_suffix(".so.tmp")
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", str(tmp),
           *map(str, objs)]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    tmp.replace(lib)


def build(verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    _link(objs, LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Build libbsattn.so in-tree with hipcc for gfx950.

    python -m block_sparse_long_bsattn_amd.build

Every source under csrc/ is compiled and linked into one shared library next to
this file.  HIP code is built with packed-fp32 instruction generation turned off.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libbsattn.so")
SOURCES = ["abi.cpp", "layout.hip", "bs_fwd.hip", "bs_bwd.hip", "lf_fwd.hip", "lf_bwd.hip"]

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs: the softmax reads them with VALU
    # instructions, and the AGPR form costs a copy per accumulator register
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # NaN inputs give NaN outputs either way; without this every fmaxf operand is
    # canonicalised first (infinities are still honoured: masking relies on -inf)
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libbsattn.so")
    return exe


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link libbsattn.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()

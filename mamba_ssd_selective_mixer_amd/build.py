"""Compile the HIP sources under csrc/ into libssd_mi355x.so for gfx950.

Each .hip file is compiled to an object in _build/ (in parallel), then all
objects are linked into the shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libssd_mi355x.so")
CEIL_LIB = os.path.join(HERE, "libssd_ceilings.so")

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 VALU forms: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """libssd_mi355x.so from csrc/*.hip, and the benchmark's separate
    machine-ceiling library libssd_ceilings.so from csrc/ceilings/."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    csrc = os.path.join(CSRC, "ceilings", "ceilings.hip")
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        objs = list(ex.map(_compile, srcs + [csrc]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], CEIL_LIB)
    if verbose:
        print(f"built {LIB} and {CEIL_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

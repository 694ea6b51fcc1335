"""Builds the HIP library ``libmoe.so`` in-tree for gfx950.

Run as ``python -m expert_ffn_layer_router_amd.build_lib``; ``__graft_entry__.build()``
calls :func:`build`. Each ``csrc/*.hip`` file is compiled to an object under
``_build/`` (in parallel), then linked into ``expert_ffn_layer_router_amd/libmoe.so``.
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
BUILD = ROOT / "_build"
LIB = PKG / "libmoe.so"
ARCH = "gfx950"

# Packed-fp32 instructions are kept out of the generated code on purpose: hipcc -O3 would
# otherwise form them from plain float code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", str(INCLUDE), "-I", str(CSRC),
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(CSRC.glob("*.hip"))


def _compile(src: Path) -> Path:
    obj = BUILD / (src.stem + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    srcs = sources()
    workers = max(1, min(len(srcs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB.with_name(LIB.name + ".tmp")
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp),
           *map(str, objs)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

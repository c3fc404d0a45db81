"""Build liblazyattn.so in-tree with hipcc for gfx950.

Usage: ``python -m position_agnostic_paged_amd.build`` (or ``build()``).
Every translation unit is compiled to an object in ``_build/`` in parallel and
linked into ``position_agnostic_paged_amd/liblazyattn.so``.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblazyattn.so")

SOURCES = ["attention.hip", "prefill_lds.hip", "kv_write.hip", "host.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed-fp32 VALU forms are disabled for all device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-result"]
# Per-source extras.  The staged prefill never tests for NaN, so it runs with
# the IEEE mode bit off: min/max then take operands as they are instead of
# quieting each one first (infinities keep their meaning).
EXTRA = {"prefill_lds.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, "-c", *COMMON, *DEVICE_FLAGS, *EXTRA.get(src, []), path, "-o", obj]
    else:
        cmd = [HIPCC, "-c", *COMMON, "-x", "c++", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in res.stderr.splitlines() if "not a recognized feature" not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", *DEVICE_FLAGS, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)

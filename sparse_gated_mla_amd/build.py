"""Builds libsga.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python -m sparse_gated_mla_amd.build              # libsga.so
    python -m sparse_gated_mla_amd.build --timeline   # libsga_timeline.so

hipcc cross-compiles for gfx950 and needs no GPU. Packed-fp32 instructions are
switched off for all device code. The timeline library is the same sources
built with SGA_TIMELINE defined: the step's kernels also record per-workgroup
device-clock stamps, which `bench.py --timeline` reads. Nothing loads it
unless asked to.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsga.so")
TIMELINE_LIB = os.path.join(PKG, "libsga_timeline.so")
SOURCES = ["sga_api.hip", "indexer.hip", "topk.hip", "attention.hip", "cache.hip", "proj.hip",
           "measure.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def command(out: str = LIB, extra=()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}",
            *[os.path.join(CSRC, s) for s in SOURCES], *extra, "-o", out]


def build(verbose: bool = False, timeline: bool = False) -> str:
    """Compiles every HIP source into libsga.so next to this file (or, with
    timeline, into libsga_timeline.so with the device-clock stamps); returns its path."""
    lib = TIMELINE_LIB if timeline else LIB
    tmp = lib + ".tmp"
    cmd = command(tmp, ("-DSGA_TIMELINE",) if timeline else ())
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{proc.stdout}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, timeline="--timeline" in sys.argv))

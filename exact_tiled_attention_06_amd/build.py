"""Build libfa.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

Usage: ``python -m exact_tiled_attention_06_amd.build`` (or ``build()`` from
Python).  The library is written next to this file, so it travels with the
source tree.
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "fa_fwd.hip")]
HEADERS = [os.path.join(HERE, "csrc", f) for f in ("fa_common.hpp", "fa_mfma.hpp", "fa_split.hpp", "fa_ksplit.hpp", "fa_f32m.hpp", "fa_bwd.hpp", "fa_window.hpp", "fa_split_window.hpp")] + [
    os.path.join(ROOT, "include", "fa.h")]
LIBRARY = os.path.join(HERE, "libfa.so")
# the instruction-rate microbenchmarks (a measurement tool, separate library)
MICRO_SOURCE = os.path.join(HERE, "csrc", "fa_micro.hip")
MICRO_LIBRARY = os.path.join(HERE, "libfa_micro.so")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms stay off: plain fp32 arithmetic only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no NaN ever enters the kernels (masked scores are -inf, never NaN), so the
    # max reductions need no NaN canonicalisation; the host checks test bits
    "-fno-honor-nans",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the HIP library)")


def _compile(sources, output: str, verbose: bool) -> None:
    tmp = output + ".tmp"
    cmd = [hipcc(), *FLAGS, "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-8000:]}")
    os.replace(tmp, output)


def build(verbose: bool = False) -> str:
    """Compile every HIP source: LIBRARY (the attention kernels and their C ABI)
    and MICRO_LIBRARY (the microbenchmarks); always recompiles."""
    _compile(SOURCES, LIBRARY, verbose)
    _compile([MICRO_SOURCE], MICRO_LIBRARY, verbose)
    return LIBRARY


def source_hash() -> str:
    """sha256 over every source and header the library is built from, plus the
    compiler flags: a profile taken of one build is valid for another build
    only when this matches."""
    h = hashlib.sha256()
    for f in SOURCES + HEADERS:
        with open(f, "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(FLAGS).encode())
    return h.hexdigest()


def is_stale() -> bool:
    if not os.path.exists(LIBRARY):
        return True
    t = os.path.getmtime(LIBRARY)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    path = build(verbose=True)
    print(path)
    sys.exit(0)

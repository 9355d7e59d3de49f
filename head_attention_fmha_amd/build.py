"""Compile the HIP sources into head_attention_fmha_amd/libfmha.so for gfx950.

Run as `python -m head_attention_fmha_amd.build`.  hipcc cross-compiles, so
this works on a machine without a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libfmha.so")
SOURCES = [os.path.join(CSRC, "fmha_api.hip")]
# attainable-peak probes used by the benchmark (not the attention path)
PEAKS_LIB_PATH = os.path.join(PKG, "libfmha_peaks.so")
PEAKS_SOURCES = [os.path.join(PKG, "peaks", "peaks.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(sources, out_path, include_dirs, verbose):
    tmp = out_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed fp32 VALU ops stay disabled: the compiler must not emit them
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function",
           *[a for d in include_dirs for a in ("-I", d)],
           *sources, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in res.stderr.splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out_path)
    return out_path


def build_library(verbose: bool = False) -> str:
    """The attention library, then the attainable-peak probes."""
    _compile(SOURCES, LIB_PATH, [os.path.join(ROOT, "include"), CSRC], verbose)
    _compile(PEAKS_SOURCES, PEAKS_LIB_PATH, [os.path.join(ROOT, "include")], verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))

"""Ahead-of-time build of the HIP library libfm.so for gfx950.

``python -m stft_mel_spectrogram_amd.build`` (or ``build()``) compiles every
source under ``csrc/`` with hipcc into ``stft_mel_spectrogram_amd/libfm.so``,
in place, so the shared object ships with the source tree.  It always
recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfm.so")
SOURCES = ["fm_api.cpp", "fm_plan.cpp", "fm_kernels.hip"]

# Packed-FP32 VALU forms are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    exe = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return exe


def build(verbose: bool = False, arch: str = "gfx950") -> str:
    """Compile libfm.so for `arch`; returns its path.  Raises on failure."""
    fd, tmp = tempfile.mkstemp(suffix=".so", prefix=".libfm-", dir=PKG)
    os.close(fd)
    cmd = [hipcc(), f"--offload-arch={arch}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-command-line-argument", *DEVICE_FLAGS,
           "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr[-8000:]}")
        if verbose and r.stderr.strip():
            print(r.stderr[-4000:], file=sys.stderr)
        os.replace(tmp, LIB)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

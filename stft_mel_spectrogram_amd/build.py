"""Ahead-of-time build of the HIP library libfm.so for gfx950.

``python -m stft_mel_spectrogram_amd.build`` (or ``build()``) compiles every
source under ``csrc/`` with hipcc (one translation unit per FFT shape, in
parallel) and links ``stft_mel_spectrogram_amd/libfm.so`` in place, so the
shared object ships with the source tree.  It always recompiles.
"""
from __future__ import annotations

import glob
import os
import re
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfm.so")
SOURCES = ["fm_api.cpp", "fm_plan.cpp", "fm_launch.hip"]


def sources() -> list:
    """Host/ABI sources plus one fm_shape_<n1>x<n2>.hip per built FFT shape,
    one fm_large_<a>x<c>x<d>.hip per large-FFT shape and one
    fm_pair_<r>x<r>.hip per paired-kernel shape."""
    def units(pattern):
        return sorted(os.path.basename(f) for f in glob.glob(os.path.join(CSRC, pattern)))
    return SOURCES + units("fm_shape_*.hip") + units("fm_large_*.hip") + units("fm_pair_*.hip")

# Packed-FP32 VALU forms are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Kernels must not use scratch (private) memory: on the MI355X a launch of a
# kernel with any scratch costs about 20 us (2.4 us without), more than the
# whole forward pass, so a register spill is a build error.  The compiler's
# resource remarks report the scratch size of every kernel.
RESOURCE_FLAGS = ["-Rpass-analysis=kernel-resource-usage"]
_REMARK_NAME = re.compile(r"remark:\s+Function Name: (\S+)")
_REMARK_SCRATCH = re.compile(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)")


def scratch_users(stderr: str) -> list:
    """(kernel, bytes per lane) for every kernel whose remarks report scratch."""
    out, name = [], None
    for line in stderr.splitlines():
        m = _REMARK_NAME.search(line)
        if m:
            name = m.group(1)
            continue
        m = _REMARK_SCRATCH.search(line)
        if m and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def hipcc() -> str:
    exe = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return exe


def build(verbose: bool = False, arch: str = "gfx950", jobs: int = 0) -> str:
    """Compile libfm.so for `arch`; returns its path.  Raises on failure."""
    common = [f"--offload-arch={arch}", "-O3", "-std=c++17", "-fPIC", "-Wall",
              "-Wno-unused-command-line-argument", *DEVICE_FLAGS, "-I", INCLUDE, "-I", CSRC]
    tmpdir = tempfile.mkdtemp(prefix=".libfm-build-", dir=PKG)
    fd, tmp = tempfile.mkstemp(suffix=".so", prefix=".libfm-", dir=PKG)
    os.close(fd)
    try:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
            extra = RESOURCE_FLAGS if src.endswith(".hip") else []
            cmd = [hipcc(), *common, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src} ({r.returncode}):\n{r.stderr[-8000:]}")
            spills = scratch_users(r.stderr)
            if spills:
                raise RuntimeError(f"{src}: kernels use scratch memory (register spills), "
                                   f"which costs ~20 us per launch: {spills}")
            if verbose and r.stderr.strip():
                print("\n".join(l for l in r.stderr.splitlines() if "kernel-resource-usage" not in l)[-4000:],
                      file=sys.stderr)
            return obj

        srcs = sources()
        n = jobs or min(len(srcs), max(1, min(os.cpu_count() or 1, 16)))
        with ThreadPoolExecutor(max_workers=n) as ex:
            objs = list(ex.map(compile_one, srcs))
        cmd = [hipcc(), f"--offload-arch={arch}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc link failed ({r.returncode}):\n{r.stderr[-8000:]}")
        os.replace(tmp, LIB)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

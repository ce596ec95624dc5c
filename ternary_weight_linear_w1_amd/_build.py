"""Compile the HIP sources into ``libbitlinear.so`` (in-tree) with hipcc for gfx950, and the
benchmark's calibration kernels into ``libbitlinear_peaks.so``."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbitlinear.so")
SOURCES = [os.path.join(CSRC, "bitlinear_api.hip")]
DEPS = SOURCES + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")] + [
    os.path.join(os.path.dirname(HERE), "include", "bitlinear.h")]
PEAKS_LIB = os.path.join(HERE, "libbitlinear_peaks.so")
PEAKS_SOURCES = [os.path.join(CSRC, "peaks.hip")]
PEAKS_DEPS = PEAKS_SOURCES

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # IEEE fp32 division and no contraction: codes depend on exact fp32 products/quotients
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep packed-fp32 instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def _compile(sources, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *sources, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    if verbose and r.stderr:
        print(r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _compile(SOURCES, LIB, verbose)
    _compile(PEAKS_SOURCES, PEAKS_LIB, verbose)
    return LIB


def _newer_than(out, deps) -> bool:
    if not os.path.exists(out):
        return False
    t = os.path.getmtime(out)
    return all(os.path.getmtime(p) <= t for p in deps)


def up_to_date() -> bool:
    """Both libraries exist and are newer than every source they are built from."""
    return _newer_than(LIB, DEPS) and _newer_than(PEAKS_LIB, PEAKS_DEPS)


if __name__ == "__main__":
    print(build(verbose=True))

"""Build the HIP library in-tree with hipcc for gfx950.

    python -m exact_attention_65_amd.build        # writes exact_attention_65_amd/libfa_mi355x.so

The library is the C ABI of include/fa.h: the host validation (pure C++) and
the launcher + kernels (HIP).  It is built for gfx950 only.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = [os.path.join(CSRC, "fa_check.cpp"), os.path.join(CSRC, "fa_fwd.hip"), os.path.join(CSRC, "fa_bwd.hip"),
           os.path.join(CSRC, "fa_fp8.hip")]
# measurement probes for the benchmark (clock stamps, MFMA loop): a library of
# their own, so the attention ABI carries nothing but the attention
PROBE_LIB_PATH = os.path.join(PKG, "libfa_probe_mi355x.so")
PROBE_SOURCES = [os.path.join(CSRC, "fa_probe.hip")]
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled for all device code.  The kernels'
# slot loops must unroll completely (their fragment arrays then live in
# registers); at head dimension 256 they exceed the default size limit of an
# unroll requested by pragma, and the arrays fall back to scratch memory.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-pragma-unroll-threshold=1000000"]
COMMON = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC] + DEVICE_FLAGS


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build the library")


def _link(sources, path: str, verbose: bool) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc()] + COMMON + ["-fPIC", "-shared", "-fvisibility=hidden"] + sources + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile the attention library and the probe library; returns the
    attention library's path.  Always recompiles."""
    _link(SOURCES, LIB_PATH, verbose)
    _link(PROBE_SOURCES, PROBE_LIB_PATH, verbose)
    return LIB_PATH


def device_asm(source: str = "fa_fwd.hip") -> str:
    """gfx950 assembly of one source file (device code only), for inspection in tests."""
    cmd = [hipcc()] + COMMON + ["--cuda-device-only", "-S", os.path.join(CSRC, source), "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed:\n{r.stderr}")
    return r.stdout


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

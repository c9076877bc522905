"""Builds the HIP library libmqa_fp4.so in-tree for gfx950 (hipcc, no GPU needed)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmqa_fp4.so")
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("mqa_kernels.hip", "mqa_api.hip", "mqa_quant.hip", "mqa_decode.hip")]
# measurement probes (bench only), a library of their own beside the operator's
PROBE_LIB = os.path.join(PKG, "libmqa_fp4_probe.so")
PROBE_SOURCES = [os.path.join(PKG, "csrc", "mqa_probe.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms stay disabled on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _build_one(lib: str, sources, verbose: bool) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Builds the operator library and the bench-only probe library."""
    _build_one(LIB, SOURCES, verbose)
    _build_one(PROBE_LIB, PROBE_SOURCES, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

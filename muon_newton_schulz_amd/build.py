"""Build libmuon.so (gfx950 only) in-tree with hipcc.

    python -m muon_newton_schulz_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmuon.so")
SOURCES = ["muon_abi.hip", "elementwise.hip", "ns_gemm.hip", "ns_f32.hip", "ns_small.hip", "guard.hip",
           "clip.hip"]
# stand-alone measurement programs: the GPU's sustained bf16 MFMA rate and
# its HBM stream rates
PROGRAMS = [("mfma_ceiling", "mfma_ceiling.hip"), ("hbm_ceiling", "hbm_ceiling.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _hipcc(cmd, out, verbose):
    tmp = out + ".tmp"
    cmd = [*cmd, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    _hipcc([HIPCC, *FLAGS, *srcs], LIB, verbose)
    exe_flags = [f for f in FLAGS if f not in ("-fPIC", "-shared")]
    for exe, src in PROGRAMS:
        _hipcc([HIPCC, *exe_flags, os.path.join(CSRC, src)], os.path.join(PKG, exe), verbose)
    return LIB


if __name__ == "__main__":
    build()

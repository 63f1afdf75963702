"""Builds libswinattn.so in-tree with hipcc for gfx950.

Usage: ``python shifted_window_attention_swin_amd/build.py`` (run it by path:
importing the package itself requires the built library).  Every HIP source
is compiled with packed FP32 instructions disabled (``-packed-fp32-ops``);
hipcc's host pass warns that it does not know that feature, which is
harmless.  ``-fno-honor-nans``: inputs are required to be finite (NaN inputs
give unspecified results), which lets max reductions skip NaN quieting.
``-amdgpu-mfma-vgpr-form``: MFMA results stay in VGPRs, where the softmax
reads them, instead of round-tripping through AGPRs.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libswinattn.so")
SOURCES = ["swinattn_api.hip", "wattn_kernels.hip", "wattn_persistent.hip", "linear_gemm.hip",
           "wattn_backward.hip", "ln_qkv_wattn.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libswinattn)")


def command(out: str = LIB, extra=()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", *extra, "-o", out,
            *[os.path.join(CSRC, s) for s in SOURCES]]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Test support: the LDS scrubber (``lds_scrub.hip``), built by
``__graft_entry__.build()`` into ``libldsscrub.so`` beside its source."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lds_scrub.hip")
LIB = os.path.join(HERE, "libldsscrub.so")


def build_lds_scrub() -> str:
    hipcc = os.environ.get("HIPCC") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        hipcc = shutil.which("hipcc") or hipcc
    tmp = LIB + ".tmp"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O2", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-o", tmp, SRC], check=True, capture_output=True, text=True)
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lds_scrub(seed: int, stream: int, blocks: int = 2048) -> None:
    """Queues the scrub on `stream` (a raw hipStream_t address)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is missing: run __graft_entry__.build()")
        _lib = ctypes.CDLL(LIB)
        _lib.lds_scrub.argtypes = [ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p]
        _lib.lds_scrub.restype = ctypes.c_int
    rc = _lib.lds_scrub(seed & 0xFFFFFFFF, blocks, stream)
    if rc != 0:
        raise RuntimeError(f"lds_scrub failed: {rc}")

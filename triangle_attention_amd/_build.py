"""Compile the gfx950 HIP library libtriattn.so in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SRCS = [os.path.join(PKG_DIR, "csrc", f) for f in ("tri_attn.hip", "tri_mul.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libtriattn.so")

# Packed FP32 VALU forms are switched off for the device code; hipcc's host pass warns that
# it does not know the feature, which is harmless.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the gfx950 library cannot be built")


def build(verbose: bool = False, extra_flags=()) -> str:
    """Always recompiles; writes the library atomically and returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, *SRCS, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    log = "\n".join(x for x in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in x)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{log}")
    if verbose and log.strip():
        print(log)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH

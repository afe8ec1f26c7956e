"""Builds libmamba2scan.so (the HIP kernels plus the C ABI) for gfx950, in-tree.

    python -m bwd_mamba2_scan_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SRC = os.path.join(PKG_DIR, "csrc", "mamba2_scan.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmamba2scan.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # Keep the compiler from emitting packed fp32 (v_pk_*_f32) instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile the library; returns its path.  Raises on compiler failure."""
    tmp = f"{LIB_PATH}.tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    out = "\n".join(ln for ln in proc.stdout.splitlines() if noise not in ln)
    if proc.returncode != 0:
        if os.path.exists(tmp):
            os.unlink(tmp)
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{out}")
    if out.strip() and verbose:
        print(out, flush=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

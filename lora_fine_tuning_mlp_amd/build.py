"""Build the HIP library (liblora_mi355x.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "lora_mi355x.hip")
HEADERS = [os.path.join(PKG, "csrc", f) for f in ("common.h", "gemm.h", "kernels_fwd.h", "kernels_bwd.h")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblora_mi355x.so")
ARCH = "gfx950"     # MI355X (CDNA4) only


def hipcc_command(out: str) -> list:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    return [
        hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # Packed fp32 VALU forms stay off (the compiler still vectorises the rest).
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", os.path.join(PKG, "csrc"),
        SRC, "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile the library every time it is called; returns the .so path."""
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Builds libadaflash.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libadaflash.so")
SOURCES = ["adaflash_kernels.hip", "adaflash_length_head.hip", "adaflash_api.cpp", "adaflash_layout.cpp",
           "adaflash_admission.cpp", "adaflash_noalloc.hip"]

# Packed-FP32 VALU instructions are disabled for every HIP translation unit.
# A local that shadows another is an error (a shadowed call epoch once tagged
# the row-barrier records with the wrong value).
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    "-Werror=shadow",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc] + HIPCC_FLAGS + ["-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that line.
    msgs = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and "--hip-link" not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))

"""Builds libadaflash.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import re
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libadaflash.so")
SOURCES = ["adaflash_kernels.hip", "adaflash_length_head.hip", "adaflash_api.cpp", "adaflash_layout.cpp",
           "adaflash_admission.cpp", "adaflash_noalloc.hip"]

# Packed-FP32 VALU instructions are disabled for every HIP translation unit.
# A local that shadows another is an error (a shadowed call epoch once tagged
# the row-barrier records with the wrong value).  The compiler reports each
# kernel's register and scratch use, and a kernel with a private (scratch)
# segment or spilled vector registers fails the build: the row kernels are
# sized to keep their chunks in registers, and an instance that once spilled
# chunk words left gradient entries unwritten from call to call.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    "-Werror=shadow",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Rpass-analysis=kernel-resource-usage",
]


def scratch_users(remarks: str) -> list[tuple[str, str, int]]:
    """(kernel, what, amount) for every kernel whose resource-usage remarks
    show a scratch segment or spilled VGPRs (SGPR spills go to VGPR lanes,
    not memory, and are allowed)."""
    out, kernel = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            kernel = m.group(1)
            continue
        for what, pat in (("scratch bytes per lane", r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)"),
                          ("spilled VGPRs", r"remark:\s+VGPRs Spill: (\d+)")):
            m = re.search(pat, line)
            if m and int(m.group(1)) > 0:
                out.append((kernel or "?", what, int(m.group(1))))
    return out


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc] + HIPCC_FLAGS + ["-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature;
    # drop that line and the resource remarks (with their source echo).
    msgs, in_remark = [], False
    for line in res.stderr.splitlines():
        if "kernel-resource-usage" in line:
            in_remark = True
            continue
        if in_remark and re.match(r"^\s*\d*\s*\|", line):
            continue
        in_remark = False
        if "packed-fp32-ops" not in line and "--hip-link" not in line:
            msgs.append(line)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    bad = scratch_users(res.stderr)
    if bad:
        raise RuntimeError("kernels with scratch memory or spilled registers:\n" +
                           "\n".join(f"  {k}: {w} {n}" for k, w, n in bad))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))

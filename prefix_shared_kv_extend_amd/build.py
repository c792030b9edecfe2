"""Build librax.so in-tree: host radix tree (C++17) + gfx950 HIP kernels, one shared library.

    python -m prefix_shared_kv_extend_amd.build      # or __graft_entry__.build()

hipcc cross-compiles for gfx950 without a GPU. Every HIP source goes through one
device translation unit (csrc/kernels/librax.hip). Packed-fp32 VALU ops are
disabled for the device code (the host pass warns that it does not know the
feature; that is harmless).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "librax.so")
ARCH = os.environ.get("RAX_OFFLOAD_ARCH", "gfx950")

SOURCES = [
    os.path.join(CSRC, "kernels", "librax.hip"),
    os.path.join(CSRC, "radix_tree.cpp"),
    os.path.join(CSRC, "rax_api.cpp"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build librax)")


SANITIZED_LIB = os.path.join(PKG, "librax_san.so")
# host code only: AddressSanitizer and UndefinedBehaviorSanitizer on the tree, the API and
# the launch code; the device code is built as usual
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SANITIZED_LIB if sanitize else LIB
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O1" if sanitize else "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-mllvm", "-amdgpu-kernarg-preload-count=14",
           "-Wall", "-Wno-unused-function",
           *(SANITIZE_FLAGS if sanitize else []),
           *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"librax build failed:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))

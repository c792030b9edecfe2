"""The host tree under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

    python -m prefix_shared_kv_extend_amd.sanitize_check

Builds librax_san.so (host code of the tree, the C API and the launch code instrumented;
device code as usual), then runs the tree, host-tier and scheduler tests against it in a
child process with the sanitizer runtime preloaded: every radix-tree operation those tests
drive (random operation sequences checked against the oracle model, host-tier moves,
scheduler batches) runs instrumented. Any report fails the run (UBSan stops on the first
error, ASan on the first invalid access). Exit status: the child's.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from .build import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = ["tests/test_abi_tree.py", "tests/test_host_tier.py", "tests/test_scheduler.py"]


def asan_runtime() -> str:
    found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("the clang AddressSanitizer runtime of ROCm's compiler was not found")
    return found[-1]


def main() -> int:
    lib = build(verbose=False, sanitize=True)
    env = dict(os.environ)
    pre = asan_runtime()
    env["LD_PRELOAD"] = pre + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["RAX_LIB_PATH"] = lib
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", *TESTS]
    print("sanitized library:", lib, flush=True)
    print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


if __name__ == "__main__":
    sys.exit(main())

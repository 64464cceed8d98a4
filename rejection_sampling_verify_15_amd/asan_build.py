"""Debug build of the library's host code with AddressSanitizer.

    python -m rejection_sampling_verify_15_amd.asan_build

Compiles every csrc/*.hip for gfx950 with AddressSanitizer on the host pass
only (the device code is built as usual), into
_asan/libspecverify_host_asan.so.  It serves the CPU tests of the
C-ABI argument checks, workspace queries and status tables: load it with the
ASan runtime preloaded (asan_runtime()) and select it for the binding with
SV_LIBRARY=<path>.
"""
from __future__ import annotations

import os
import subprocess
import sys

from .build import ARCH, CSRC, INCLUDE, hipcc, sources

HERE = os.path.dirname(os.path.abspath(__file__))
ASAN_LIB = os.path.join(HERE, "_asan", "libspecverify_host_asan.so")


def asan_runtime() -> str:
    """Path of clang's AddressSanitizer runtime that matches hipcc."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/lib/llvm/bin/clang"
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    if out.returncode != 0 or not os.path.exists(path):
        raise RuntimeError("clang's AddressSanitizer runtime was not found")
    return path


def up_to_date() -> bool:
    """The ASan build exists and is newer than every source it is built from."""
    if not os.path.exists(ASAN_LIB):
        return False
    t = os.path.getmtime(ASAN_LIB)
    deps = sources() + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")]
    deps.append(os.path.join(INCLUDE, "specverify.h"))
    return all(os.path.getmtime(d) <= t for d in deps)


def build_host_asan(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(ASAN_LIB), exist_ok=True)
    tmp = ASAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-fvisibility=hidden", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
           "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC, "-o", tmp] + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{proc.stdout}")
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    print(build_host_asan(verbose="-v" in sys.argv))

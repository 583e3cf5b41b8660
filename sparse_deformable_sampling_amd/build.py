"""Build libdcn.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdcn.so")
ROOT = os.path.dirname(HERE)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # fp32 atomicAdd lowers to the hardware global atomic, not a CAS loop
    "-munsafe-fp-atomics",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libdcn.so (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-o", tmp] + sources()
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def build_sanitized(path: str) -> str:
    """The same library with AddressSanitizer and UndefinedBehaviorSanitizer in
    its host code only (argument checks, planning, launch set-up); the device
    code is built as usual.  A process loads it with the compiler's
    libclang_rt.asan preloaded and LIBDCN_PATH=path."""
    host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-shared-libsan"]
    subprocess.check_call([HIPCC] + flags + host + ["-I", os.path.join(ROOT, "include"), "-o", path] + sources())
    return path


def sanitizer_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (it carries the
    UndefinedBehaviorSanitizer handlers too)."""
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return found[-1]


if __name__ == "__main__":
    print(build(verbose=True))

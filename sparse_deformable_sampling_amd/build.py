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


# The debug build: the same sources with every forward output store counted
# (DCN_COUNT_WRITES; include/dcn_debug.h).  Only the tests load it.
COUNT_LIB = os.path.join(HERE, "libdcn_count.so")
BUILD_DIR = os.path.join(HERE, "_build")


def _compile_link(lib: str, defines: list, verbose: bool) -> str:
    """Compile each source to an object (in parallel), then link lib."""
    from concurrent.futures import ThreadPoolExecutor
    tag = "count" if defines else "prod"
    os.makedirs(BUILD_DIR, exist_ok=True)
    cflags = [f for f in FLAGS if f != "-shared"] + defines + ["-I", os.path.join(ROOT, "include"), "-c"]
    jobs = []
    for src in sources():
        obj = os.path.join(BUILD_DIR, "%s.%s.%d.o" % (os.path.basename(src)[:-4], tag, os.getpid()))
        jobs.append(([HIPCC] + cflags + ["-o", obj, src], obj))
    if verbose:
        for cmd, _ in jobs:
            print(" ".join(cmd), file=sys.stderr)
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "0")) or os.cpu_count() or 1, 16))
    tmp = lib + ".tmp%d" % os.getpid()
    try:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda j: subprocess.check_call(j[0]), jobs))
        subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for _, o in jobs])
        os.replace(tmp, lib)
    finally:
        for f in [o for _, o in jobs] + [tmp]:
            if os.path.exists(f):
                os.remove(f)
    return lib


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libdcn.so, and the write-counting debug
    build libdcn_count.so (always recompiles both)."""
    _compile_link(LIB, [], verbose)
    _compile_link(COUNT_LIB, ["-DDCN_COUNT_WRITES"], verbose)
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

"""The oracle and the host side of libdcn under AddressSanitizer and
UndefinedBehaviorSanitizer: both are rebuilt with the sanitizers (the C
oracle whole, libdcn's host code only -- argument checks, planning, launch
set-up), and tests/test_oracle.py and tests/test_abi.py run against those
builds in a child process with the sanitizer runtime preloaded.  Any report
fails the run (UBSan is built not to recover, ASan halts on its first error).
CPU only: no kernel is launched."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle
from sparse_deformable_sampling_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def tools_present():
    try:
        libbuild.sanitizer_runtime()
    except FileNotFoundError:
        return False
    return os.path.exists(libbuild.HIPCC) and os.path.exists("/opt/rocm/llvm/bin/clang") and shutil.which("nm")


def undefined_symbols(path):
    out = subprocess.run(["nm", "-D", "--undefined-only", path], capture_output=True, text=True, check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if line.strip()}


@pytest.mark.skipif(not tools_present(), reason="hipcc, clang or the clang sanitizer runtime is missing")
def test_oracle_and_abi_tests_pass_under_asan_and_ubsan(tmp_path):
    lib = libbuild.build_sanitized(str(tmp_path / "libdcn_san.so"))
    orc = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    # both builds call into the sanitizer runtime
    for path in (lib, orc):
        syms = undefined_symbols(path)
        assert any(s.startswith("__asan_report_") for s in syms), path
        assert any(s.startswith("__ubsan_handle_") for s in syms), path

    env = dict(os.environ)
    env.update(LD_PRELOAD=libbuild.sanitizer_runtime(), LIBDCN_PATH=lib, ORACLE_LIB_PATH=orc,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", PYTHONDONTWRITEBYTECODE="1")
    # the child process maps the sanitized builds, not the default ones
    probe = ("import oracle; from sparse_deformable_sampling_amd import _binding as B; oracle._load(); B.lib(); "
             "print(open('/proc/self/maps').read())")
    maps = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=300)
    assert maps.returncode == 0, maps.stderr[-3000:]
    for path in (lib, orc, libbuild.sanitizer_runtime()):
        assert os.path.realpath(path) in maps.stdout, path

    run = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle.py", "tests/test_abi.py", "-q", "-x",
                          "-m", "not gpu", "-p", "no:cacheprovider"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    text = run.stdout + run.stderr
    assert "AddressSanitizer" not in text, text[-6000:]
    assert "runtime error:" not in text, text[-6000:]
    assert run.returncode == 0, text[-6000:]
    assert " passed" in run.stdout, text[-3000:]

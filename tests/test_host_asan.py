"""The C-ABI's host code under AddressSanitizer (CPU only): the host-only
ASan build of the library runs the argument checks, workspace queries,
status tables and test controls of test_abi.py in a child process with the
ASan runtime preloaded; any ASan report fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_code_under_asan():
    from rejection_sampling_verify_15_amd import asan_build
    try:
        runtime = asan_build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = asan_build.ASAN_LIB if asan_build.up_to_date() else asan_build.build_host_asan()
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True)
    assert "__asan_init" in nm.stdout or "__asan_report" in nm.stdout, "the build is not instrumented"
    env = dict(os.environ)
    env.update(SV_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=0:halt_on_error=1",
               PYTHONDONTWRITEBYTECODE="1")
    probe = subprocess.run([sys.executable, "-c", "print('libclang_rt.asan' in open('/proc/self/maps').read())"],
                           env=env, capture_output=True, text=True, timeout=120)
    assert probe.stdout.strip() == "True", probe.stdout + probe.stderr
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                           os.path.join(ROOT, "tests", "test_abi.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = proc.stdout + proc.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert proc.returncode == 0, out[-4000:]
    assert " passed" in out

"""The C ABI host layer under AddressSanitizer (CPU): the library is built a second time
with ASan on its host code (device code unchanged), and tests/test_abi.py runs against that
build with the ASan runtime preloaded. Every call there goes through the host-side checks,
error strings, workspace-size queries and the profiling bookkeeping; an invalid host memory
access aborts the run with an AddressSanitizer report."""
import os
import subprocess
import sys

import pytest

from learned_context_ranking_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale():
    if not os.path.exists(build_lib.ASAN_LIB):
        return True
    t = os.path.getmtime(build_lib.ASAN_LIB)
    srcs = [os.path.join(build_lib.CSRC, f) for f in os.listdir(build_lib.CSRC)]
    srcs.append(os.path.join(ROOT, "include", "sas.h"))
    return any(os.path.getmtime(p) > t for p in srcs)


@pytest.mark.timeout(900)
def test_abi_tests_under_asan():
    try:
        rt = build_lib.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    if _stale():
        build_lib.build_asan()
    # the build is instrumented (ASan report hooks referenced by the host code)
    syms = subprocess.run(["nm", "-D", build_lib.ASAN_LIB], capture_output=True, text=True).stdout
    assert "__asan_report" in syms
    env = dict(os.environ, SAS_LIB=build_lib.ASAN_LIB, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out

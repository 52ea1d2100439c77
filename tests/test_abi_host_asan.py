"""The host-side C ABI checks of test_abi_host.py, run again in a child process against a build of
the library whose host code is compiled with AddressSanitizer (validation, workspace sizing and
carving, the status and error strings). No GPU is needed: every call there returns before any
launch. Any sanitizer report fails the test."""
import os
import subprocess
import sys

import pytest

from mixture_experts_layer_10_amd import build as BUILD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def asan_lib():
    try:
        BUILD.hipcc()
        runtime = BUILD.asan_runtime()
    except RuntimeError as e:
        pytest.skip(f"no HIP toolchain with a sanitizer runtime here: {e}")
    return BUILD.build_host_asan(), runtime


def test_abi_host_under_address_sanitizer(asan_lib):
    lib, runtime = asan_lib
    env = dict(os.environ, MOE_LIB_PATH=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86")
    # the child loads the sanitizer build, with the runtime in the process
    probe = ("import ctypes; from mixture_experts_layer_10_amd import binding as B; B.load(); "
             "assert B.LIB_PATH == %r; ctypes.CDLL(None).__asan_report_load8; print('asan-ok')" % lib)
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "asan-ok" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out

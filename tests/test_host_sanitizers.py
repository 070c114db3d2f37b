"""The library's host-side argument checking (configuration and codebook
checks, the quantizer's cell table, decode geometry and workspace sizing)
runs the whole ABI test module clean under AddressSanitizer and
UndefinedBehaviorSanitizer.  Host code only: the device objects are the
ordinary build's.  CPU only; nothing is launched."""

import os
import shutil
import subprocess
import sys

import pytest

from compressed_space_attention_isoquant_amd import build as Bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _available():
    try:
        Bd._rocm_clang()
        Bd.hostsan_runtime()
        return True
    except Exception:
        return False


@pytest.mark.skipif(not _available(), reason="ROCm clang++ or its ASan runtime is missing")
def test_abi_module_clean_under_asan_and_ubsan():
    lib = Bd.build_host_sanitized()
    # the library really is instrumented
    if shutil.which("nm"):
        syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ)
    env.update({
        "IQ_TEST_LIBRARY": lib,
        "LD_PRELOAD": Bd.hostsan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-m", "not gpu", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout

"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle (hs_oracle.c), the input generator (fill.c) and the host side of
libhisparse (argument checks, handles, launch planning; the device code is
built as always) are compiled with ASan + UBSan, every check fatal, into a
temporary directory. A child process that preloads the sanitizer runtime
then runs the oracle's pins, the input-generator tests and the C-ABI checks
against those builds (HS_ORACLE_LIB, HS_INPUTS_LIB, HS_LIB). No GPU is
needed: the library's host checks run without one.
"""
import os
import subprocess
import sys

import pytest

import oracle
from tiered_kv_cache_hs_amd import build as B
from tiered_kv_cache_hs_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUNTIME = os.path.join(os.path.dirname(oracle.SAN_CC), "..", "lib", "clang")


def _asan_runtime():
    for dirpath, _, files in os.walk(RUNTIME):
        if "libclang_rt.asan-x86_64.so" in files:
            return os.path.join(dirpath, "libclang_rt.asan-x86_64.so")
    return None


@pytest.mark.slow
def test_host_code_clean_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None or not os.path.exists(oracle.SAN_CC):
        pytest.skip("no clang sanitizer runtime in this image")
    out = str(tmp_path)
    env = dict(os.environ)
    env["HS_ORACLE_LIB"] = oracle.build_sanitized(out)
    env["HS_INPUTS_LIB"] = I.build_sanitized(out, oracle.SAN_CC, oracle.SAN_FLAGS,
                                             oracle.SAN_LINK)
    env["HS_LIB"] = B.build_host_sanitized(out)
    env["LD_PRELOAD"] = rt
    # python itself is not instrumented: its allocations are not leaks to report
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=87"
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           "tests/test_oracle_resolve.py", "tests/test_oracle_attention.py",
           "tests/test_oracle_batch.py", "tests/test_inputs.py", "tests/test_abi.py",
           "tests/test_policy_sim.py", "-m", "not gpu and not slow"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    log = r.stdout + r.stderr
    assert "AddressSanitizer" not in log and "runtime error:" not in log, log[-4000:]
    assert r.returncode == 0, log[-4000:]
    assert " passed" in log

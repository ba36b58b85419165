"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Builds the library's host sources (the metadata builder, the layer plan and
cache estimate, the error reporting) and the oracle with g++/gcc and
-fsanitize=address,undefined (no recovery: the first report aborts), then runs
the CPU tests that exercise them, in a child pytest with the sanitizer
runtimes preloaded: the metadata against the oracle's brute force on every
workload shape and the random sweeps (300 ring/length cases, 200 with sinks,
300 rings with sinks), the cache estimator, and every oracle pin.  Any
out-of-bounds access, use after free, overflow or other undefined behaviour
fails the run.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_sliding_window_swa_amd", "csrc")
HOST_SOURCES = ["blockmask.cpp", "cache_plan.cpp", "swa_error.cpp"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _runtime(name):
    return subprocess.check_output(["gcc", "-print-file-name=" + name], text=True).strip()


@pytest.fixture(scope="module")
def sanitized_libs(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("san"))
    host = os.path.join(d, "libswa_host_san.so")
    # the HIP headers are included for their types only; no device code here
    subprocess.check_call(
        ["g++", "-std=c++17", "-shared", "-fPIC"] + SAN +
        ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
         "-I" + CSRC] + [os.path.join(CSRC, f) for f in HOST_SOURCES] + ["-o", host])
    orc = os.path.join(d, "libswa_oracle_san.so")
    subprocess.check_call(["gcc", "-std=c99", "-shared", "-fPIC", "-fno-fast-math",
                           "-ffp-contract=off"] + SAN +
                          [os.path.join(ROOT, "oracle", "swa_oracle.c"), "-o", orc, "-lm"])
    return host, orc


def test_host_code_under_sanitizers(sanitized_libs):
    host, orc = sanitized_libs
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join([_runtime("libasan.so"), _runtime("libubsan.so")])
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=97"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=98"
    env["SWA_TEST_SANITIZED_HOST_LIB"] = host
    env["SWA_TEST_SANITIZED_ORACLE_LIB"] = orc
    tests = [os.path.join(ROOT, "tests", t) for t in
             ("test_blockmask.py", "test_cache_estimator.py", "test_oracle_pins.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + tests, cwd=ROOT, env=env, capture_output=True,
                       text=True)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail
    assert "runtime error" not in tail, tail

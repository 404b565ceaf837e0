"""libdpnorm's host layer under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU.

tests/hostcheck/build.py compiles the library's sources host-only with both
sanitizers and links them against a host-side stand-in for the HIP runtime
(tests/hostcheck/fake_hip.cpp: launches only check their configuration,
nothing touches a device). Then:
  * tests/hostcheck/fuzz_plan.cpp drives every entry point with seeded random
    sizes, layer counts up to 2^20, shared inputs, short workspaces,
    misaligned and overlapping outputs; a call must agree with its workspace
    query, every launch configuration must be valid, and the sanitizers must
    stay silent (they abort the run on any finding);
  * tests/test_abi.py runs against the sanitized library through ctypes,
    with the sanitizer runtime preloaded into Python.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "hostcheck"))

import build as hostcheck_build  # noqa: E402  (tests/hostcheck/build.py)


@pytest.fixture(scope="module")
def hostcheck(tmp_path_factory):
    return hostcheck_build.build(str(tmp_path_factory.mktemp("hostcheck")))


def test_library_is_instrumented(hostcheck):
    syms = subprocess.run(["nm", "-D", "--undefined-only", hostcheck["lib"]], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms
    # the stand-in, not the HIP runtime, provides the launches
    defined = subprocess.run(["nm", "-D", "--defined-only", hostcheck["lib"]], capture_output=True, text=True).stdout
    assert "hipLaunchKernel" in defined


def test_plan_fuzz_under_sanitizers(hostcheck):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([hostcheck["fuzz"], "1000", "20261202"], capture_output=True, text=True, timeout=900,
                         env=env)
    print(res.stdout.strip(), flush=True)
    assert res.returncode == 0, res.stdout + res.stderr[-4000:]
    assert " 0 bad launches, 0 failures" in res.stdout


def test_abi_tests_under_sanitizers(hostcheck):
    env = dict(os.environ, LD_PRELOAD=hostcheck["asan_runtime"], ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", DPNORM_TEST_LIB=hostcheck["lib"])
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(HERE, "test_abi.py")], capture_output=True, text=True, timeout=900, env=env,
                         cwd=os.path.dirname(HERE))
    print(res.stdout.strip().splitlines()[-1] if res.stdout.strip() else "", flush=True)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]

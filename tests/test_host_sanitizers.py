"""The host side of the C ABI (argument checks, plans, the host arithmetic of
the cost model and the topology checks) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven by the host tests: no sanitizer report,
every test passing. CPU only; the device code is built as usual and never
runs here."""

import os
import shutil
import subprocess
import sys

import pytest

from tree_attention_verification_ancestor_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_abi_host.py", "tests/test_cost_model_host.py"]


def test_host_abi_under_address_and_undefined_behaviour_sanitizers():
    runtime = libbuild.sanitizer_runtime()
    if runtime is None or shutil.which(libbuild.HIPCC) is None and not os.path.exists(libbuild.HIPCC):
        pytest.skip("no hipcc or sanitizer runtime")
    lib = libbuild.build_sanitized()
    # the build really is instrumented
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms
    env = dict(os.environ, LD_PRELOAD=runtime, TAV_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *HOST_TESTS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert " passed" in r.stdout, report

"""The host code of libgdn (argument checks, workspace sizing, dispatch, the
allocation-free entry point's host side and the host DRRQR selector) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU: the host ABI
tests and the DRRQR host tests run in a child process against a library
whose host objects are instrumented (device code is not), with the
sanitizer runtime preloaded; any report aborts the child."""

import os
import subprocess
import sys

import pytest

from gated_deltanet_recurrent_delta_amd import build_hostsan as hs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(hs.runtime() is None, reason="no AddressSanitizer runtime")
def test_host_code_under_asan_and_ubsan():
    lib = hs.build()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms, "host objects not instrumented"
    env = dict(os.environ, LD_PRELOAD=hs.runtime(), GDN_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = subprocess.run(
        [sys.executable, "-c", "from gated_deltanet_recurrent_delta_amd import binding as b; "
                               "print(b.LIB_PATH)"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.strip() == lib
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
         "tests/test_abi_host.py", "tests/test_drrqr_host.py"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]

"""The host code of libdion3 under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/test_abi.py (argument validation, workspace planning of single calls
and of the whole step, canonical sizes, k = ceil(f n), status strings, the
teardown call) runs in a child process against the host-sanitizer build, with
the ASan runtime preloaded; any report aborts the child and fails this test.
CPU only: none of these calls reaches the GPU."""

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_abi_checks_under_host_sanitizers():
    from muon_momentum_amd import build_sanitized as S

    lib = S.build_sanitized()
    # the build really is instrumented
    und = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert re.search(r"__asan_report_(load|store)", und) and "__ubsan_handle_" in und
    env = dict(os.environ)
    env.update({"DION3_LIB": lib, "LD_PRELOAD": S.asan_runtime(),
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert re.search(r"\d+ passed", out), out[-2000:]

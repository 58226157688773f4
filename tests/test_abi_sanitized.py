"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer: the ABI tests
(test_abi_host.py), the launch-failure tests (test_abi_hooks.py) and the launch-plan
invariants (test_plans_host.py) run in a child Python
against a host-only build of the library with both sanitizers and the test hook
(build.build_check), with the sanitizer runtime preloaded.  Any sanitizer report aborts the
child, which fails this test."""
import os
import subprocess
import sys

import pytest

from indexed_sparse_attention_ix_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not available")
def test_abi_tests_pass_under_asan_and_ubsan():
    lib = B.build_check()
    env = dict(os.environ)
    env.update(IX_LIB=lib, LD_PRELOAD=B.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi_host.py", "tests/test_abi_hooks.py",
                        "tests/test_plans_host.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "skipped" not in out.splitlines()[-1], out[-2000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]

"""The C-ABI tests run against the host-sanitizer build of the library
(AddressSanitizer + UndefinedBehaviorSanitizer on api.cpp and noalloc.cpp,
launchers stubbed out by csrc/host_stubs.cpp), in a child process with the
ASan runtime preloaded. Any sanitizer report aborts the child and fails this
test. CPU only; the sanitized library is built by __graft_entry__.build()
(or `python -m paged_kv_attn_amd.build --host-sanitized`)."""

import os
import subprocess
import sys

import pytest

from paged_kv_attn_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_sanitizers():
    if not os.path.exists(B.ASAN_OUT):
        pytest.skip("host-sanitizer build not present (built by __graft_entry__.build())")
    env = dict(os.environ)
    env.update(LD_PRELOAD=B.asan_runtime(), ATTN_LIBRARY=B.ASAN_OUT,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_binding_checks.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout, tail

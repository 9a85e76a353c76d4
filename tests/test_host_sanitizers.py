"""The C ABI's host logic under AddressSanitizer and UndefinedBehaviorSanitizer.

libevoattn_asan.so is the library with its host code (argument and layout
checks, alias checks, workspace planning, the launch sequences, the profiling
records) built with -fsanitize=address,undefined; its device code is that of
the plain build.  The C-ABI tests that need no GPU run against it in a child
interpreter with clang's ASan runtime preloaded, halting on the first report.
"""
import os
import subprocess
import sys

import pytest

from evoformer_biased_attention_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = """
import sys
sys.path.insert(0, {root!r})
from evoformer_biased_attention_amd import _lib
_lib.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu", {tests!r}]))
"""


@pytest.mark.timeout(900)
def test_abi_host_logic_under_asan_and_ubsan():
    if not B.ASAN_RUNTIME:
        pytest.skip("clang's ASan runtime is not installed")
    if B.asan_is_stale():
        B.build_asan()
    code = _CHILD.format(root=ROOT, lib=B.LIB_ASAN, tests=os.path.join(ROOT, "tests", "test_abi.py"))
    env = dict(os.environ, LD_PRELOAD=B.ASAN_RUNTIME, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail

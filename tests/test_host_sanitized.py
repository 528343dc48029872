"""The host-only tests (the host-backed plane store, the expert caches,
routing, the bit allocator, argument validation) rerun against libpm_asan.so,
whose host code is built with AddressSanitizer and UndefinedBehaviorSanitizer
(halting on the first report), in a child process that preloads the ASan
runtime."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from bitplane_quantized_expert_amd import build  # noqa: E402

SOURCES = build.TARGETS[0][1]


def test_host_code_under_asan_and_ubsan():
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("no ASan runtime next to hipcc")
    lib = build.ASAN_LIB
    newest = max(os.path.getmtime(s) for s in SOURCES)
    if not os.path.exists(lib) or os.path.getmtime(lib) < newest:
        build.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=rt, PM_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", "tests/test_host_abi.py", "tests/test_cache.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout, out

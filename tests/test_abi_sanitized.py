"""The C ABI's host code (argument validation, workspace sizing, dispatch) built with
AddressSanitizer and UndefinedBehaviorSanitizer, with every ABI test run against it in a child
process that preloads the sanitizer runtime.  CPU only: no kernel is launched."""
import os
import subprocess
import sys

import pytest

from gated_linear_attention_chunkwise_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))


def test_abi_tests_pass_under_host_sanitizers():
    try:
        so = build.build_host_sanitized()
        rt = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(f"sanitized build unavailable: {e}")
    pre = os.environ.get("LD_PRELOAD")
    env = dict(os.environ, LD_PRELOAD=rt + (":" + pre if pre else ""),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", LIZARD_ATTN_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py")], env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert r.returncode == 0, out[-3000:]
    assert "Sanitizer" not in out and "runtime error" not in out
    assert "passed" in out

"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A host-sanitized build of the library (tests/sanitized_build.py) runs the
whole CPU ABI suite (tests/test_abi_cpu.py: every host validation code,
workspace sizing and layout, the 32-bit tile limits, batch 0) in a child
process with the sanitizer runtime preloaded.  Any invalid access or
undefined operation in the argument checks or the layout arithmetic aborts
that run (cudnn-frontend PR #462, "Why this was never caught (commit 2)": a
sizing bug that writes out of bounds stays silent without such a check).
No kernel is launched.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.timeout(600)
def test_abi_suite_under_host_sanitizers():
    try:
        import sanitized_build as sb  # noqa: F401  (tests/ is on sys.path under pytest)
    except ImportError:
        sys.path.insert(0, HERE)
        try:
            import sanitized_build as sb
        except ImportError:
            pytest.skip("the sanitizer build helper is not present in this copy")
    from variable_length_attention_ragged_amd import build as b
    if not shutil.which(b.hipcc()) and not os.path.exists(b.hipcc()):
        pytest.skip("hipcc not available")
    try:
        lib = sb.build()
        rt = sb.runtime()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "VARLEN_ATTN_LIBRARY": lib,
    })
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "-m", "not gpu", os.path.join(HERE, "test_abi_cpu.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=540)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out

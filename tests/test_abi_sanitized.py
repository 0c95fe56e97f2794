"""The C-ABI tests again, against a build of the library whose host code runs
under AddressSanitizer and UndefinedBehaviorSanitizer (the device code is
built as usual and never launched: these calls make no GPU work). A memory
error or undefined behaviour in the argument checks, the workspace layout or
the plan objects aborts the child process, so the test fails."""
import os
import subprocess
import sys

import pytest

from permuted_block_sparse_amd import build as sa_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_host_sanitizers(tmp_path):
    try:
        sa_build.hipcc()
        runtime = sa_build.sanitizer_runtime()
    except RuntimeError as err:
        pytest.skip(str(err))
    lib = sa_build.build(out=str(tmp_path / "libsparse_attn_sanitized.so"),
                         sanitize=True)
    env = dict(os.environ)
    env.update({
        "SPARSE_ATTN_LIB": lib,
        "LD_PRELOAD": runtime,
        # the interpreter's own allocations are not this library's
        "ASAN_OPTIONS": "detect_leaks=0",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_abi.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "passed" in out and "AddressSanitizer" not in out, out[-4000:]

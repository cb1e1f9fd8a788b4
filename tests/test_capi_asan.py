"""The C ABI's host code under AddressSanitizer (CPU only).

The host side of libw4a4 (argument validation, size queries, error
messages, the launch wrappers) is rebuilt with AddressSanitizer
(`build.build_asan`; device code unchanged), the sanitizer runtime is
preloaded into a fresh python process, and test_capi_cpu.py runs against
that library: every validation path and size query must pass with no
sanitizer report."""
import os
import subprocess
import sys

import pytest

from w4a4_block_scaled_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))


def test_capi_validation_under_address_sanitizer():
    try:
        runtime = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = B.build_asan(jobs=8)
    env = dict(os.environ, LD_PRELOAD=runtime, W4A4_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    probe = ("import ctypes, w4a4_block_scaled_amd as w4; L = w4.lib(); "
             "assert w4.library_path() == %r; "
             "assert hasattr(ctypes.CDLL(None), '__asan_init'); print('asan ok')" % lib)
    chk = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True,
                         timeout=300, cwd=os.path.dirname(HERE))
    assert "asan ok" in chk.stdout, chk.stdout[-2000:] + chk.stderr[-2000:]
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(HERE, "test_capi_cpu.py")],
                         env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout[-4000:] + res.stderr[-4000:]
    assert res.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in res.stderr, out
    assert " passed" in res.stdout

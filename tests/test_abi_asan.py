"""The C ABI's host code under AddressSanitizer: the library is rebuilt with
its host side (argument validation, split plans, launch set-up) sanitized,
and every CPU test of the ABI runs against it in a process with the
sanitizer runtime preloaded.  Any invalid access aborts that process.  No
kernel is launched.  CPU only."""
import os
import shutil
import subprocess
import sys

import pytest

from quantized_kv_cache_token_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))


def test_abi_host_code_is_clean_under_address_sanitizer():
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime next to the compiler")
    lib = build.build_asan()
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               LD_LIBRARY_PATH=os.path.dirname(rt) + ":" + os.environ.get("LD_LIBRARY_PATH", ""))
    r = subprocess.run([sys.executable, os.path.join(HERE, "native", "abi_under_asan.py"), lib], env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.strip().startswith("ran ") and int(r.stdout.split()[-1]) >= 15

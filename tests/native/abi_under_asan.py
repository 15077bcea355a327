"""Runs every test of tests/test_abi_cpu.py against the library whose host
code is built with AddressSanitizer (argv[1]); the sanitizer runtime is
preloaded by the caller.  Prints the number of tests run."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from quantized_kv_cache_token_amd import lkv  # noqa: E402

lkv.LIB_PATH = sys.argv[1]
from tests import test_abi_cpu as T  # noqa: E402

n = 0
for name in sorted(dir(T)):
    if name.startswith("test_") and callable(getattr(T, name)):
        getattr(T, name)()
        n += 1
print("ran", n, flush=True)

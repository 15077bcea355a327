"""MI355X-native quantised KV-cache decode attention (K6/V4).

The compute path is a HIP library for gfx950 behind a C ABI
(include/lkv.h); `quantized_kv_cache_token_amd.lkv` is its thin ctypes
binding.  PyTorch only provides device memory and streams.
"""

"""SemKV mixed-precision KV-cache hot path for MI355X (gfx950).

The compute lives in libsemkv.so (HIP kernels behind the C ABI of
include/semkv.h); `kv_cache_mixed_top_amd.semkv` is its thin Python binding.
Importing the binding fails loudly if the library has not been built.
"""

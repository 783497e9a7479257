"""TurboQuant KV-cache compression and attention over the packed cache,
native to AMD Instinct MI355X (gfx950).

The hot path lives in libtq.so (HIP kernels + C ABI, include/tq.h);
``kv_cache_vector_compress_amd.tq`` is its thin Python binding and
``kv_cache_vector_compress_amd.synth`` holds the seeded input generators.
"""

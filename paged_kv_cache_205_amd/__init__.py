"""MI355X (gfx950) paged decode attention and one-token KV append.

The compute lives in the HIP library ``libpa.so`` (C ABI declared in
``include/pa.h``); ``paged_kv_cache_205_amd.ops`` is a thin ctypes binding over
it that only marshals torch tensors into pointers and the current HIP stream.
``paged_kv_cache_205_amd.synth`` draws the seeded synthetic workloads.
"""

"""MI355X-native chunked-prefill attention over a paged KV cache.

The compute lives in libpaged_kv_prefill.so (hand-written gfx950 HIP kernels
behind a C ABI, declared in include/paged_kv_prefill.h).  `ops` is the thin
ctypes binding with the same entry-point names; `synth` makes seeded inputs.
Submodules are imported on use: `from paged_kv_prefill_amd import ops`.
"""

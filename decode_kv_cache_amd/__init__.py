"""MI355X-native Kara window-compression step: score -> Token2Chunk select -> paged compaction.

The compute runs in ``libkara.so`` (hand-written HIP kernels for gfx950 behind
a C ABI declared in ``include/kara.h``); ``decode_kv_cache_amd.kara`` is the thin
ctypes binding, ``decode_kv_cache_amd.workloads`` makes seeded synthetic inputs.
"""

"""MI355X-native speculative verification step over a hierarchical sparse KV cache.

The work is done by libkvhier.so (HIP kernels for gfx950 behind the C ABI of
``include/kv_hier.h``); this package holds its sources (``csrc/``), the build
script and a thin ctypes binding.
"""
from .binding import (  # noqa: F401
    EXPORTED, KV_EWAIT, KV_FLAG_POISON, KV_FLAG_SERIAL, KV_FLAG_SYNC_BACKUP, KV_FLAG_TEST_FAIL_ATTN, KV_FLAG_TIMING,
    KV_FLAG_TIMING_ATTN, KV_TIER_HOT, KV_TIER_RESIDENT, KV_TIER_RING, KV_TIER_STAGED, KVHier, KVHierError, LIB_PATH,
    load_library, loc_code,
)

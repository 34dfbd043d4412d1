"""MI355X-native query-free KV-cache eviction step.

* ``kv_cache_token_amd.api`` -- the C ABI of libkvevict (include/kvevict.h) with
  the same names: qf_score_keys, kv_evict_topk, kv_compact_gather,
  kv_evict_one_inplace, qf_filters_load / save / from_queries / from_keys,
  kvx_stats.
* ``kv_cache_token_amd.cache.EvictingCache`` -- buffers + offset bookkeeping for
  a model's (layer, batch, KV head) groups, one ``update`` per incoming block.
* ``kv_cache_token_amd.synth`` -- seeded synthetic inputs.

Importing the package loads nothing; the library is loaded on first use and its
absence is an error.
"""

__all__ = ["api", "cache", "synth", "build"]

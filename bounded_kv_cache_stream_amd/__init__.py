"""Bounded streaming KV cache for MI355X: paged frame-to-cache attention and
cache management (page write, sliding-window eviction, CLCES score and top-k
compaction, diversity-scored per-head pruning) in hand-written HIP kernels
behind a C ABI (include/kvstream.h).

``kvstream`` is the ctypes binding; ``synth`` generates the seeded workloads;
``build`` compiles the library in-tree.
"""

from .kvstream import (  # noqa: F401
    KV_BF16, KV_FP32, KV_TRANSIENT, KVCache, KVError, kv_append_attend, kv_append_frame, kv_append_frame_layers,
    kv_diversity_prune, kv_diversity_prune_layers, kv_diversity_score, kv_diversity_score_layers, kv_evict,
    kv_get_head_lengths, kv_get_info, kv_get_page_table, kv_last_error, kv_layer_budgets, kv_merge_pages,
    kv_merge_pages_layers,
    kv_pool_create, kv_pool_destroy, kv_pool_get_layout, kv_pool_required_bytes, kv_reset, kv_set_attend_splits,
    make_config, score_and_compact, stream_attend, kv_sync, KV_CLCES_DEFER,
)

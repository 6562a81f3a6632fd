"""softmax_attention_amd: grouped-query softmax attention forward for MI355X.

The computation runs in libmiattn.so (hand-written HIP kernels for gfx950,
C ABI in include/miattn.h); this package is its thin Python binding plus the
seeded synthetic workload generators.
"""
from .binding import (MiattnError, attn_bwd, attn_fwd_dense, attn_fwd_paged, attn_fwd_paged_append,
                      attn_fwd_paged_varlen, attn_fwd_varlen, kv_cache_write, lib,
                      profile_start, profile_stop, release_workspace, set_split_keys,
                      set_streamk_piece, attn_fwd_paged_noalloc)

__all__ = ["MiattnError", "attn_bwd", "attn_fwd_dense", "attn_fwd_paged", "attn_fwd_paged_append",
           "attn_fwd_paged_varlen", "attn_fwd_varlen", "kv_cache_write", "lib", "profile_start",
           "profile_stop", "release_workspace", "set_split_keys", "set_streamk_piece",
           "attn_fwd_paged_noalloc"]

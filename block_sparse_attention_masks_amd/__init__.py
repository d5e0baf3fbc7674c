"""Block-sparse softmax attention over 3D video tokens on AMD MI355X (gfx950).

The calls of libvsa (tile reorder; STA / radial / NABLA block masks and their
composition; SICS block scores; KV-cache compaction; block-sparse attention
forward, also on raster-order tokens with the tiles as blocks or grouped across
frames, and backward), bound with ctypes; torch supplies device memory and streams.  See include/vsa.h for the C ABI.
"""
from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, VSA_BF16, VSA_F32, VsaError, all_ones_mask, ar_forced_ranges, lib,
    nabla_workspace_bytes, sta_capacity, status_string, vsa_block_sparse_attn_fwd, vsa_block_sparse_attn_bwd,
    attn_bwd_workspace_bytes, attn_fwd_workspace_bytes, vsa_tiled_attn_fwd, tiled_attn_workspace_bytes,
    vsa_radial_attn_fwd, attn_fwd_workspace_bytes_radial, vsa_block_sparse_attn_fwd_static,
    vsa_mask_nabla, vsa_mask_radial, vsa_mask_sta, vsa_tile_reorder,
    sta_heads_capacity, vsa_mask_sta_heads, vsa_mask_union, vsa_block_sics, vsa_block_mean_pool,
    compact_tokens, vsa_kv_compact, vsa_kv_gather, vsa_kv_plan, vsa_mask_remap,
)

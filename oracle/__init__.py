"""fp64 CPU oracle of the block-sparse 3D-video attention path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import or call anything in this package; the
product path (the HIP library and its binding) never does, and shares no code,
table or helper with it.  Inputs come from the seeded generators in `workloads`.

Every function here is the plain definition of what the path computes, written
from the pages, step by step, in fp64 (numpy):

  reorder.tile_reorder   -- 3D tiles made contiguous (Sliding Tile Attention
                            explainer, aibr.jp/archives/60739, sec. 2-3)
  masks.mask_sta         -- sliding 3D tile window (same page, sec. 3)
  masks.mask_radial      -- energy-decay radial mask (Radial Attention explainer,
                            aibr.jp/archives/112136, sec. 2-3)
  masks.mask_nabla       -- pooled-map CDF threshold mask (NABLA explainer,
                            aibr.jp/archives/124678, sec. 1 and 3)
  masks.mask_ar          -- anchors + recent + selected blocks (Sparse Forcing
                            summary, gist.science/ja/paper/2604.21221, part 2)
  masks.mask_sta_heads   -- STA with a window per head (STA explainer, sec. 1)
  masks.mask_union       -- union of two masks, e.g. NABLA with STA (NABLA
                            explainer, sec. 2 and 4)
  sics.block_sics        -- SPADE's sum of intra-block cosine similarities
                            (SPADE summary, gist.science/ja/paper/2608.03335)
  kvcache.kv_keep / kv_compact / mask_remap
                         -- KV-cache compaction to the kept blocks (Sparse
                            Forcing summary, parts 2-3)
  attention.attention    -- exact softmax(Q K^T * scale) V over the kept blocks
  attention.attention_bwd-- its gradients dQ, dK, dV (chain rule, step by step)

Where the pages leave a step open, the reading taken is stated in the function.
"""
from .reorder import tile_reorder, tile_order_source  # noqa: F401
from .masks import (  # noqa: F401
    csr_from_bool, csr_to_bool, mask_all, mask_sta, mask_radial, radial_keep_tokens,
    pool_blocks, nabla_select_row, mask_nabla, ar_forced_ranges, ar_select_row, mask_ar, pooled_maps,
    nabla_cut_admissible, topk_admissible, forced_flags,
    mask_sta_heads, mask_union, csr_concat,
)
from .attention import (  # noqa: F401
    attention, attention_bwd, attention_bwd_key_block, attention_bwd_query_rows, attention_rows, block_softmax,
)
from .sics import block_sics  # noqa: F401
from . import kvcache  # noqa: F401

"""The synthetic workloads, as plain data (shapes, dtypes, seeds, mask knobs).

Nothing here computes any part of the method; both the fp64 oracle and the GPU
path read these numbers. Each workload is named by what it is:

  tiny   -- 2 heads, head_dim 64, fp32, 8x16x16 grid (2,048 tokens), 4x4x4 tiles
            (32 blocks of 64); run with an all-ones mask, an STA window of 1x3x3
            tiles and a NABLA mask at CDF threshold 0.9.
  sta    -- 24 heads, head_dim 128, bf16, 30x48x80 grid (115,200 tokens), 6x8x8
            tiles (384 tokens, 5x6x10 tile grid), 3x3x5 tile window clipped at the
            grid border (Sliding Tile Attention explainer, aibr.jp/archives/60739,
            sec. 3).
  nabla  -- 40 heads, head_dim 128, bf16, 16x48x80 grid (61,440 tokens), 1x8x8 tiles
            (960 blocks of 64), CDF threshold 0.8 (NABLA explainer,
            aibr.jp/archives/124678, sec. 3).
  radial -- 24 heads, head_dim 128, bf16, 125x45x80 grid (450,000 tokens, 3,600 per
            frame), raster order, 128-token blocks (Radial Attention explainer,
            aibr.jp/archives/112136, sec. 3).
  ar     -- 12 heads, head_dim 128, bf16; a 3-frame query chunk of 3x30x52 (4,680
            tokens) = frames 18..20 of a 21-frame KV cache of 21x30x52 (32,760
            tokens), 64-token raster blocks; anchors (frame 0) + the last 3 frames +
            the top-16 other blocks per query block (Sparse Forcing summary,
            gist.science/ja/paper/2604.21221, part 2).
  nabla_sta -- the nabla workload with the NABLA mask united with a 3x3x5 STA
            window on its 16x6x10 tile grid (NABLA explainer, sec. 2 and 4).
  sta_heads -- the sta workload with a window per head, cycling 3x3x5, 1x3x3,
            3x5x7 over the heads (STA explainer, sec. 1: heads specialise).
  ar_compact -- the ar workload with its KV cache compacted to the blocks each
            head keeps before attention (Sparse Forcing summary, parts 2-3).

Value model (synthetic stand-in for model activations; the pages give no
statistics): Q = a*N(0,1) + P, K = a*N(0,1) + P, V = c*N(0,1) (+ P for `ar`), where
P is a per-head positional code 1.5*[cos, sin](w_j . (t, h, w)) with 64 frequency
vectors w_j ~ U[-0.6, 0.6]^3 per head.  It imitates the 3D locality described in
the Sliding Tile Attention explainer, sec. 1 and 3.
"""

CONFIGS = {
    "tiny": dict(
        seed=1, batch=1, heads=2, head_dim=64, dtype="f32",
        grid=(8, 16, 16), tile=(4, 4, 4),
        qk_noise=1.0, positional=False, v_positional=False,
        sta_window=(1, 3, 3), nabla_threshold=0.9,
    ),
    "sta": dict(
        seed=2, batch=1, heads=24, head_dim=128, dtype="bf16",
        grid=(30, 48, 80), tile=(6, 8, 8), window=(3, 3, 5),
        qk_noise=0.5, positional=True, v_positional=False,
    ),
    "nabla": dict(
        seed=3, batch=1, heads=40, head_dim=128, dtype="bf16",
        grid=(16, 48, 80), tile=(1, 8, 8), threshold=0.8,
        qk_noise=0.5, positional=True, v_positional=False,
    ),
    "radial": dict(
        seed=4, batch=1, heads=24, head_dim=128, dtype="bf16",
        grid=(125, 45, 80), block=128,
        qk_noise=0.5, positional=True, v_positional=False,
    ),
    # Mask composition on the NABLA and STA inputs (same seeds, hence the same tensors).
    "nabla_sta": dict(
        seed=3, batch=1, heads=40, head_dim=128, dtype="bf16",
        grid=(16, 48, 80), tile=(1, 8, 8), threshold=0.8, window=(3, 3, 5),
        qk_noise=0.5, positional=True, v_positional=False,
    ),
    "sta_heads": dict(
        seed=2, batch=1, heads=24, head_dim=128, dtype="bf16",
        grid=(30, 48, 80), tile=(6, 8, 8), windows=((3, 3, 5), (1, 3, 3), (3, 5, 7)),
        qk_noise=0.5, positional=True, v_positional=False,
    ),
    "ar": dict(
        seed=5, batch=1, heads=12, head_dim=128, dtype="bf16",
        grid=(21, 30, 52),            # the KV cache
        q_frames=(18, 21),            # the query chunk = frames [18, 21) of the cache
        block=64, topk=16, anchor_frames=1, recent_frames=3,
        qk_noise=1.0, positional=True, v_positional=True,
    ),
}

# The ar chunk with its KV cache compacted to the blocks each head keeps (same inputs).
CONFIGS["ar_compact"] = dict(CONFIGS["ar"])


def n_tokens(grid):
    t, h, w = grid
    return t * h * w


def q_grid(cfg):
    """Token grid of the queries (the chunk for `ar`, the full grid otherwise)."""
    if "q_frames" in cfg:
        f0, f1 = cfg["q_frames"]
        return (f1 - f0, cfg["grid"][1], cfg["grid"][2])
    return cfg["grid"]


def q_frame_offset(cfg):
    return cfg["q_frames"][0] if "q_frames" in cfg else 0

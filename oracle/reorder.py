"""Tile reorder (oracle).

Sliding Tile Attention explainer (aibr.jp/archives/60739), sec. 2-3: the video is
cut into small rectangular 3D tiles and attention is organised per tile, so that a
tile's tokens are handled as one unit; the SPADE summary (gist.science/ja/paper/
2608.03335, "The solution", part 1) describes the same T x H x W grid cut into
slices.  Reading taken: tiles of tt x th x tw tokens over a T x H x W grid that
each tile size divides; tiles are ordered in raster order over the tile grid, and
tokens inside a tile in raster order.
"""
import numpy as np


def tile_order_source(grid, tile):
    """src[p] = raster token index of the token placed at tile-major position p."""
    T, H, W = grid
    tt, th, tw = tile
    if T % tt or H % th or W % tw:
        raise ValueError("grid not divisible by tile")
    NH, NW = H // th, W // tw
    V = tt * th * tw
    p = np.arange(T * H * W, dtype=np.int64)
    tile_id, r = p // V, p % V
    it, ih, iw = tile_id // (NH * NW), (tile_id // NW) % NH, tile_id % NW
    lt, lh, lw = r // (th * tw), (r // tw) % th, r % tw
    t, h, w = it * tt + lt, ih * th + lh, iw * tw + lw
    return (t * H + h) * W + w


def tile_reorder(x, grid, tile, inverse=False):
    """Permute the token axis (axis 1) of x [B, N, ...]: raster -> tile-major, or
    back with inverse=True."""
    src = tile_order_source(grid, tile)
    out = np.empty_like(x)
    if inverse:
        out[:, src] = x
    else:
        out[:] = x[:, src]
    return out

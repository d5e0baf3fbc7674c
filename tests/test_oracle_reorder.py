"""Pins of the oracle's tile reorder (CPU only)."""
import itertools

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")

GRIDS = [((8, 16, 16), (4, 4, 4)), ((30, 48, 80), (6, 8, 8)), ((16, 48, 80), (1, 8, 8)),
         ((4, 6, 10), (2, 3, 5)), ((3, 5, 7), (1, 1, 1)), ((2, 2, 2), (2, 2, 2))]


@pytest.mark.parametrize("grid,tile", GRIDS)
def test_bijection_and_inverse(grid, tile):
    src = oracle.tile_order_source(grid, tile)
    n = int(np.prod(grid))
    assert np.array_equal(np.sort(src), np.arange(n))
    x = np.random.default_rng(0).standard_normal((2, n, 3))
    y = oracle.tile_reorder(x, grid, tile)
    assert np.array_equal(oracle.tile_reorder(y, grid, tile, inverse=True), x)


@pytest.mark.parametrize("grid,tile", GRIDS)
def test_matches_reshape_transpose(grid, tile):
    """Independent formulation: split each axis into (tile index, in-tile index) and
    move all tile indices in front of all in-tile indices."""
    T, H, W = grid
    tt, th, tw = tile
    x = np.random.default_rng(1).standard_normal((2, T * H * W, 2, 3))
    ref = (x.reshape(2, T // tt, tt, H // th, th, W // tw, tw, 2, 3)
           .transpose(0, 1, 3, 5, 2, 4, 6, 7, 8).reshape(2, T * H * W, 2, 3))
    assert np.array_equal(oracle.tile_reorder(x, grid, tile), ref)


def test_bruteforce_positions():
    """Walk every token of a small grid by hand and place it."""
    grid, tile = (4, 6, 10), (2, 3, 5)
    T, H, W = grid
    tt, th, tw = tile
    NH, NW = H // th, W // tw
    V = tt * th * tw
    src = oracle.tile_order_source(grid, tile)
    for t, h, w in itertools.product(range(T), range(H), range(W)):
        tile_id = ((t // tt) * NH + h // th) * NW + w // tw
        inner = ((t % tt) * th + h % th) * tw + w % tw
        assert src[tile_id * V + inner] == (t * H + h) * W + w


def test_rejects_non_divisible():
    with pytest.raises(ValueError):
        oracle.tile_order_source((5, 4, 4), (2, 2, 2))

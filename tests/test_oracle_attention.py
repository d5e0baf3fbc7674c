"""Pins of the oracle's attention and of the input generator (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from workloads import gen
from workloads.configs import CONFIGS


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_attention_golden(golden_dir):
    with open(os.path.join(golden_dir, "attention_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        k = np.array(c["k"], dtype=np.float64).reshape(1, -1, 1, 1)
        v = np.array(c["v"], dtype=np.float64).reshape(1, -1, 1, 1)
        q = np.array(c["q"]).reshape(1, 1, 1, 1)
        nkb = -(-k.shape[1] // 2)
        keep = np.zeros((1, nkb), dtype=bool)
        keep[0, c["kept"]] = True
        rp, ci = oracle.csr_from_bool(keep)
        o, lse = oracle.attention(q, k, v, rp, ci, 1, 2, 1.0)
        assert o[0, 0, 0, 0] == pytest.approx(c["o"], abs=1e-14)
        want = {"ln4": math.log(4.0), "-inf": -math.inf}[c["lse"]]
        assert lse[0, 0, 0] == pytest.approx(want, abs=1e-14) if want != -math.inf else lse[0, 0, 0] == want


@pytest.mark.parametrize("nq,nk,bq,bk", [(64, 64, 16, 16), (100, 77, 32, 16), (37, 130, 8, 64)])
def test_all_ones_equals_sdpa_fp64(nq, nk, bq, bk):
    """All-ones mask = dense attention = torch's scaled_dot_product_attention (fp64, CPU)."""
    rng = np.random.default_rng(nq)
    q, k, v = _rand(rng, 2, nq, 3, 16), _rand(rng, 2, nk, 3, 16), _rand(rng, 2, nk, 3, 16)
    rp, ci = oracle.mask_all(-(-nq // bq), -(-nk // bk))
    o, lse = oracle.attention(q, k, v, rp, ci, bq, bk, 16 ** -0.5)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v)).permute(0, 2, 1, 3).numpy()
    assert np.abs(o - ref).max() < 1e-12
    s = np.einsum("bqhd,bkhd->bhqk", q, k) * 16 ** -0.5
    assert np.abs(lse - logsumexp(s, axis=-1)).max() < 1e-12


def test_sparse_equals_bruteforce_rows():
    """Per output row, by explicit loops over the kept key tokens."""
    rng = np.random.default_rng(1)
    nq, nk, bq, bk, D = 20, 23, 4, 5, 3
    q, k, v = _rand(rng, 1, nq, 2, D), _rand(rng, 1, nk, 2, D), _rand(rng, 1, nk, 2, D)
    keep = rng.random((2 * 5, 5)) < 0.5
    keep[3] = False                                   # one empty row
    rp, ci = oracle.csr_from_bool(keep)
    o, lse = oracle.attention(q, k, v, rp, ci, bq, bk, 0.7, n_slabs=2)
    for h in range(2):
        for t in range(nq):
            r = h * 5 + t // bq
            keys = [j for j in range(nk) if keep[r, j // bk]]
            if not keys:
                assert np.all(o[0, t, h] == 0) and lse[0, h, t] == -np.inf
                continue
            s = [sum(q[0, t, h, d] * k[0, j, h, d] for d in range(D)) * 0.7 for j in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            l = sum(w)
            want = [sum(w[a] * v[0, j, h, d] for a, j in enumerate(keys)) / l for d in range(D)]
            assert np.allclose(o[0, t, h], want, atol=1e-13, rtol=0)
            assert abs(lse[0, h, t] - (m + math.log(l))) < 1e-13


def test_block_gather_equals_masked_dense():
    """Two formulations: gather the kept blocks, or mask all others with -inf."""
    rng = np.random.default_rng(2)
    nq, nk, bq, bk, D = 90, 70, 16, 8, 8
    q, k, v = _rand(rng, 1, nq, 2, D), _rand(rng, 1, nk, 2, D), _rand(rng, 1, nk, 2, D)
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    keep = rng.random((2 * nbq, nbk)) < 0.3
    keep[:, 0] = True
    rp, ci = oracle.csr_from_bool(keep)
    o, lse = oracle.attention(q, k, v, rp, ci, bq, bk, 0.3, n_slabs=2)
    for h in range(2):
        toks = np.arange(nq)
        o2, l2 = oracle.attention_rows(q[0, :, h], toks, k[0, :, h], v[0, :, h], rp, ci, h * nbq, bq, bk, 0.3)
        assert np.abs(o2 - o[0, :, h]).max() < 1e-13
        assert np.abs(l2 - lse[0, h]).max() < 1e-13


def test_rows_sum_to_one_and_constant_v():
    rng = np.random.default_rng(3)
    p = oracle.block_softmax(_rand(rng, 30, 8) * 4, _rand(rng, 50, 8) * 4, 0.5)
    assert np.abs(p.sum(axis=1) - 1).max() < 1e-12
    q, k = _rand(rng, 1, 40, 1, 8), _rand(rng, 1, 40, 1, 8)
    v = np.full((1, 40, 1, 8), 2.5)
    keep = rng.random((5, 5)) < 0.5
    keep[:, 2] = True
    o, _ = oracle.attention(q, k, v, *oracle.csr_from_bool(keep), 8, 8, 1.0)
    assert np.abs(o - 2.5).max() < 1e-13


def test_reorder_equivariance_dense():
    """Dense attention commutes with the token permutation of the tile reorder."""
    grid, tile = (4, 4, 8), (2, 2, 4)
    rng = np.random.default_rng(4)
    q, k, v = (_rand(rng, 1, 128, 2, 8) for _ in range(3))
    rp, ci = oracle.mask_all(8, 8)
    o, _ = oracle.attention(q, k, v, rp, ci, 16, 16, 0.35)
    r = lambda x: oracle.tile_reorder(x, grid, tile)
    o2, _ = oracle.attention(r(q), r(k), r(v), rp, ci, 16, 16, 0.35)
    assert np.abs(oracle.tile_reorder(o2, grid, tile, inverse=True) - o).max() < 1e-13


def test_sta_covering_window_equals_dense():
    grid, tile = (8, 16, 16), (4, 4, 4)
    rng = np.random.default_rng(5)
    q, k, v = (_rand(rng, 1, 2048, 1, 8) for _ in range(3))
    o1, _ = oracle.attention(q, k, v, *oracle.mask_sta(grid, tile, (3, 7, 7)), 64, 64, 0.35)
    o2, _ = oracle.attention(q, k, v, *oracle.mask_all(32, 32), 64, 64, 0.35)
    assert np.array_equal(o1, o2)


# ------------------------------------------------------------------ inputs
def test_positional_code_norm():
    """Sum over features of P^2 = 1.5^2 * 64 * (cos^2 + sin^2) = 144 for every token."""
    cfg = dict(CONFIGS["sta"])
    cfg["qk_noise"] = 0.0
    om = gen.omega(cfg)
    x = gen._values(cfg, "q", 0, 3, 1000, 1400, om)
    assert np.abs((x ** 2).sum(axis=1) - 144.0).max() < 1e-9


def test_generator_rounding_and_head_slices():
    x = gen.make_tensor("tiny", "v")
    assert x.dtype == torch.float32 and x.shape == (1, 2048, 2, 64)
    raw = gen._values(CONFIGS["tiny"], "v", 0, 1, 0, 2048, gen.omega("tiny"))
    assert np.array_equal(x[0, :, 1].numpy(), raw.astype(np.float32))
    ar_q = gen.make_tensor("ar", "q")
    assert ar_q.shape == (1, 4680, 12, 128) and ar_q.dtype == torch.bfloat16
    h = gen.head_values("ar", "q", 0, 7, 100, 4680)
    assert np.array_equal(h, ar_q[0, 100:, 7].double().numpy())
    rows = gen.sample_rows("sta", 4096)
    assert len(rows) == 4096 and len({tuple(r) for r in rows}) == 4096
    assert [0, 0, 115199] in rows.tolist()

"""Pins of the oracle's KV-cache compaction (CPU only).

The kept set is checked against a boolean OR of the mask rows; the compact cache
against the identity for an all-ones mask; and the whole construction against
attention: attention over the compact cache with the rewritten mask must equal
attention over the full cache with the original mask."""
import numpy as np
import pytest

import oracle
from oracle import kvcache


def _mask(rng, slabs, nbq, nbk, dens, force_tail=None):
    keep = rng.random((slabs * nbq, nbk)) < dens
    keep[:, 0] = True                                    # an anchor block in every row
    if force_tail is not None:
        keep[:, -1] = False
        for s in force_tail:
            keep[s * nbq, -1] = True                     # only these slabs keep the ragged tail
    return keep, oracle.csr_from_bool(keep)


@pytest.mark.parametrize("nk,block", [(1000, 64), (1024, 64), (333, 50)])
def test_keep_is_or_of_rows(nk, block):
    rng = np.random.default_rng(nk)
    slabs, nbq, nbk = 3, 5, -(-nk // block)
    keep, (rp, ci) = _mask(rng, slabs, nbq, nbk, 0.2)
    keeps, remap, n_full_max, has_tail = kvcache.kv_keep(rp, ci, slabs, nbq, nbk, nk, block)
    ragged = nk % block != 0
    for s in range(slabs):
        want = np.nonzero(keep[s * nbq:(s + 1) * nbq].any(axis=0))[0]
        assert np.array_equal(keeps[s], want)
        full = want[want != nbk - 1] if ragged else want
        assert np.array_equal(remap[s, full], np.arange(len(full)))
        assert np.all(remap[s, np.setdiff1d(np.arange(nbk), want)] == -1)
    assert n_full_max == max(len(k[k != nbk - 1]) if ragged else len(k) for k in keeps)


def test_all_ones_is_identity():
    rng = np.random.default_rng(1)
    nk, block = 1000, 64
    nbk = -(-nk // block)
    rp, ci = oracle.mask_all(4, nbk)
    _, remap, n_full_max, has_tail = kvcache.kv_keep(rp, ci, 1, 4, nbk, nk, block)
    n_out = kvcache.compact_tokens(n_full_max, has_tail, nk, block)
    assert n_out == nk
    x = rng.standard_normal((1, nk, 2, 8))
    assert np.array_equal(kvcache.kv_compact(x, remap, 2, block, n_out), x)


@pytest.mark.parametrize("nk,block,tail_slabs", [(1000, 64, (0, 2)), (1024, 64, None), (700, 96, (1,))])
def test_attention_over_compact_equals_full(nk, block, tail_slabs):
    rng = np.random.default_rng(nk + block)
    B, H, D, nq, bq = 1, 3, 16, 200, 50
    nbq, nbk = -(-nq // bq), -(-nk // block)
    keep, (rp, ci) = _mask(rng, B * H, nbq, nbk, 0.15, force_tail=tail_slabs if nk % block else None)
    q, k, v = (rng.standard_normal((B, n, H, D)) for n in (nq, nk, nk))
    _, remap, n_full_max, has_tail = kvcache.kv_keep(rp, ci, B * H, nbq, nbk, nk, block)
    n_out = kvcache.compact_tokens(n_full_max, has_tail, nk, block)
    assert n_out < nk
    kc = kvcache.kv_compact(k, remap, H, block, n_out)
    vc = kvcache.kv_compact(v, remap, H, block, n_out)
    rp2, ci2 = kvcache.mask_remap(rp, ci, remap, nbq)
    o_full, l_full = oracle.attention(q, k, v, rp, ci, bq, block, D ** -0.5, B * H)
    o_comp, l_comp = oracle.attention(q, kc, vc, rp2, ci2, bq, block, D ** -0.5, B * H)
    assert np.allclose(o_comp, o_full, rtol=0, atol=1e-12)
    assert np.allclose(l_comp, l_full, rtol=0, atol=1e-12)
    for r in range(len(rp2) - 1):                        # rows stay strictly ascending
        assert np.all(np.diff(ci2[rp2[r]:rp2[r + 1]]) > 0)

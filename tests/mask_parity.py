"""Comparison of a GPU block mask with the oracle's, row by row (helper of the GPU tests).

A row must match bit for bit unless the oracle flags it as one whose decision sits
within rounding of the cut:
  * CDF cut (NABLA): the running sum at the cut, or just before it, lies within 1e-5 of
    the threshold (the only rows the workloads' parity rule exempts).  Rows whose last
    kept and first dropped probabilities nearly tie are only counted: they must match.
  * top-k (AR chunk): the k-th and (k+1)-th pooled logits differ by less than 1e-5
    relative.
An exempt row that differs must still be an admissible answer, judged on the oracle's
fp64 probabilities (or logits): oracle.nabla_cut_admissible / oracle.topk_admissible.
"""
import numpy as np

import oracle


def _row(rp, ci, r):
    return ci[rp[r]:rp[r + 1]]


def compare_masks(rp, ci, orp, oci, exempt, admissible):
    """Every non-exempt row equal; every differing exempt row r passes admissible(r, kept).
    Returns (rows that differ outside the exemption, exempt rows that differ, exempt rows
    that differ and are not admissible)."""
    assert len(rp) == len(orp)
    bad, differ_ex, inadmissible = [], [], []
    for r in range(len(orp) - 1):
        got = _row(rp, ci, r)
        if np.array_equal(got, _row(orp, oci, r)):
            continue
        if not exempt[r]:
            bad.append(r)
            continue
        differ_ex.append(r)
        if not admissible(r, got):
            inadmissible.append(r)
    return bad, differ_ex, inadmissible


def _slab_map(q, k, slab, heads, block_q, block_k, scale, softmax, cache):
    """The oracle's pooled map (probabilities or logits) of one (batch, head) slab."""
    if slab not in cache:
        b, h = divmod(slab, heads)
        qs = np.asarray(q[b:b + 1, :, h:h + 1], np.float64)
        ks = np.asarray(k[b:b + 1, :, h:h + 1], np.float64)
        cache[slab] = next(oracle.pooled_maps(qs, ks, block_q, block_k, scale, softmax))
    return cache[slab]


def check_nabla(rp, ci, q, k, block_q, block_k, scale, thr, oracle_mask=None):
    """GPU CDF-cut mask (rp, ci; host arrays, one slab per (b, h)) against the oracle on q, k
    ([B, N, heads, D], the tile order the GPU pooled).  Returns a dict of counts; asserts the
    rule above."""
    heads = q.shape[2]
    nbq = -(-q.shape[1] // block_q)
    orp, oci, flagged, near_tie = (oracle.mask_nabla(q, k, block_q, block_k, scale, thr)
                                   if oracle_mask is None else oracle_mask)
    cache = {}

    def admissible(r, kept):
        p = _slab_map(q, k, r // nbq, heads, block_q, block_k, scale, True, cache)
        return oracle.nabla_cut_admissible(p[r % nbq], kept, thr)

    bad, differ_ex, inadm = compare_masks(rp, ci, orp, oci, flagged, admissible)
    counts = {"rows": len(orp) - 1, "flagged": int(flagged.sum()), "near_tie": int(near_tie.sum()),
              "near_tie_unflagged": int((near_tie & ~flagged).sum()), "flagged_differ": len(differ_ex),
              "flagged_differ_inadmissible": len(inadm), "unflagged_differ": len(bad)}
    assert not bad, f"rows differing outside the flagged set: {bad[:10]} ({counts})"
    assert not inadm, f"flagged rows whose GPU cut is not admissible: {inadm[:10]} ({counts})"
    return counts


def check_topk(rp, ci, q, k, block_q, block_k, scale, topk, forced):
    """GPU anchor + recent + top-k mask against the oracle (see check_nabla)."""
    heads = q.shape[2]
    nbq = -(-q.shape[1] // block_q)
    nbk = -(-k.shape[1] // block_k)
    orp, oci, ties = oracle.mask_ar(q, k, block_q, block_k, scale, topk, forced)
    is_forced = oracle.forced_flags(forced, nbk)
    cache = {}

    def admissible(r, kept):
        z = _slab_map(q, k, r // nbq, heads, block_q, block_k, scale, False, cache)
        return oracle.topk_admissible(z[r % nbq], kept, topk, is_forced)

    bad, differ_ex, inadm = compare_masks(rp, ci, orp, oci, ties, admissible)
    counts = {"rows": len(orp) - 1, "flagged": int(ties.sum()), "flagged_differ": len(differ_ex),
              "flagged_differ_inadmissible": len(inadm), "unflagged_differ": len(bad)}
    assert not bad, f"rows differing outside the flagged set: {bad[:10]} ({counts})"
    assert not inadm, f"flagged rows whose GPU selection is not admissible: {inadm[:10]} ({counts})"
    return counts, (orp, oci)

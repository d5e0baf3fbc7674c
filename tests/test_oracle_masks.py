"""Pins of the oracle's block masks (CPU only).

Each mask is checked against something other than itself: hand-worked golden
cases, closed forms, token-level brute force written here from the rule, and
invariants the pages fix (radial O(n log n) growth, NABLA threshold 1 keeps all)."""
import itertools
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


def rows_of(rp, ci):
    return [list(ci[rp[r]:rp[r + 1]]) for r in range(len(rp) - 1)]


# ------------------------------------------------------------------------- STA
def sta_closed_form_nnz(grid, tile, window):
    """Sum over query tiles of the clipped window volume: a product over axes of
    sum_i (min(n-1, i+h) - max(0, i-h) + 1)."""
    total = 1
    for g, t, w in zip(grid, tile, window):
        n, h = g // t, w // 2
        total *= sum(min(n - 1, i + h) - max(0, i - h) + 1 for i in range(n))
    return total


def test_sta_golden(golden_dir):
    with open(os.path.join(golden_dir, "sta_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        rp, ci = oracle.mask_sta(c["grid"], c["tile"], c["window"])
        assert rows_of(rp, ci) == c["rows"]


def test_sta_workload_counts():
    # 8x16x16 grid / 4x4x4 tiles, 1x3x3 window; 30x48x80 / 6x8x8, 3x3x5 window.
    for grid, tile, window, expect in [((8, 16, 16), (4, 4, 4), (1, 3, 3), 200),
                                       ((30, 48, 80), (6, 8, 8), (3, 3, 5), 9152)]:
        rp, ci = oracle.mask_sta(grid, tile, window)
        assert len(ci) == sta_closed_form_nnz(grid, tile, window) == expect
        lens = np.diff(rp)
        if expect == 9152:
            assert lens.min() == 12 and lens.max() == 45


@settings(max_examples=40, deadline=None)
@given(st.tuples(st.integers(1, 5), st.integers(1, 5), st.integers(1, 6)),
       st.tuples(st.integers(1, 3), st.integers(1, 3), st.integers(1, 3)),
       st.tuples(*[st.sampled_from([1, 3, 5, 7, 9, 11])] * 3))
def test_sta_closed_form_and_symmetry(ntiles, tile, window):
    grid = tuple(n * t for n, t in zip(ntiles, tile))
    rp, ci = oracle.mask_sta(grid, tile, window)
    assert len(ci) == sta_closed_form_nnz(grid, tile, window)
    keep = oracle.csr_to_bool(rp, ci, len(rp) - 1)
    assert np.array_equal(keep, keep.T)
    assert keep.diagonal().all()


def test_sta_window_covering_grid_is_dense():
    grid, tile = (8, 16, 16), (4, 4, 4)
    rp, ci = oracle.mask_sta(grid, tile, (3, 7, 7))   # >= 2n-1 tiles on every axis
    assert len(ci) == 32 * 32


def test_sta_unit_tiles_equal_token_window_bruteforce():
    """1x1x1 tiles turn the tile window into a token-level 3D sliding window."""
    grid, window = (3, 4, 5), (3, 1, 3)
    rp, ci = oracle.mask_sta(grid, (1, 1, 1), window)
    keep = oracle.csr_to_bool(rp, ci, 60)
    T, H, W = grid
    for (a, b) in itertools.product(range(60), repeat=2):
        ta, ha, wa = a // (H * W), (a // W) % H, a % W
        tb, hb, wb = b // (H * W), (b // W) % H, b % W
        want = abs(ta - tb) <= 1 and ha == hb and abs(wa - wb) <= 1
        assert keep[a, b] == want


def test_sta_rejects_bad_args():
    with pytest.raises(ValueError):
        oracle.mask_sta((8, 16, 16), (4, 4, 4), (2, 3, 3))
    with pytest.raises(ValueError):
        oracle.mask_sta((8, 16, 15), (4, 4, 4), (1, 3, 3))


# ---------------------------------------------------------------------- radial
def radial_bruteforce(T, S, block):
    """Every token pair by the rule, then lifted to blocks by 'any'."""
    N = T * S
    nb = -(-N // block)
    keep = np.zeros((nb, nb), dtype=bool)
    for qt in range(N):
        for kt in range(N):
            d = abs(qt // S - kt // S)
            r = 0
            while (2 << r) <= d:
                r += 1
            if d <= 1 or abs(qt % S - kt % S) * (1 << r) < S:
                keep[qt // block, kt // block] = True
    return keep


def test_radial_golden(golden_dir):
    with open(os.path.join(golden_dir, "radial_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        rows = rows_of(*oracle.mask_radial(c["T"], c["S"], c["block"]))
        for r, want in c["rows"].items():
            assert rows[int(r)] == want, (c["T"], c["S"], c["block"], r)


@pytest.mark.parametrize("T,S,block", [(5, 8, 2), (3, 10, 4), (9, 7, 5), (12, 16, 8),
                                       (6, 5, 13), (17, 4, 3), (1, 9, 4), (16, 20, 32)])
def test_radial_token_bruteforce(T, S, block):
    rp, ci = oracle.mask_radial(T, S, block)
    assert np.array_equal(oracle.csr_to_bool(rp, ci, len(rp) - 1), radial_bruteforce(T, S, block))


@pytest.mark.parametrize("T,S", [(9, 11), (9, 8), (17, 16)])
def test_radial_token_rule_matches_bruteforce_rule(T, S):
    # frame sizes divisible by 2^r reach the boundary |ds| * 2^r = S, which drops the pair
    n = np.arange(T * S)
    keep = oracle.radial_keep_tokens(n[:, None] // S, n[:, None] % S, n[None] // S, n[None] % S, S)
    blocks = radial_bruteforce(T, S, 1)
    assert np.array_equal(keep, blocks)


def test_radial_token_rule_boundary_pairs():
    """Hand-worked pairs at the edge of the window, S = 8 (frame, in-frame index):
    d = 2, 3 (r = 1) keep |ds| <= 3; d = 4..7 (r = 2) keep |ds| <= 1; d = 8 (r = 3) keeps
    ds = 0 only; d <= 1 keeps everything."""
    S = 8
    cases = [((0, 0), (1, 7), True), ((0, 0), (2, 3), True), ((0, 0), (2, 4), False),
             ((0, 0), (3, 3), True), ((0, 0), (3, 4), False), ((0, 0), (4, 1), True),
             ((0, 0), (4, 2), False), ((0, 7), (7, 6), True), ((0, 7), (7, 5), False),
             ((0, 3), (8, 3), True), ((0, 3), (8, 4), False), ((5, 2), (1, 3), True)]
    for (fq, sq), (fk, sk), want in cases:
        assert bool(oracle.radial_keep_tokens(fq, sq, fk, sk, S)) == want, (fq, sq, fk, sk)


def test_radial_near_frames_dense_and_single_frame():
    T, S, block = 8, 64, 16
    keep = oracle.csr_to_bool(*oracle.mask_radial(T, S, block), T * S // block)
    per = S // block
    for i in range(keep.shape[0]):
        f = i // per
        for g in range(max(0, f - 1), min(T, f + 2)):
            assert keep[i, g * per:(g + 1) * per].all()
    rp, ci = oracle.mask_radial(1, 300, 64)
    assert len(ci) == 5 * 5
    rp, ci = oracle.mask_radial(2, 300, 64)      # d <= 1 everywhere
    assert len(ci) == 10 * 10


def test_radial_n_log_n_growth():
    """Fixed S, T doubling up to 2S: kept token pairs / (N * S) grows by a constant
    per doubling (linear in log T), i.e. O(n log n) pairs, not O(n^2)."""
    S = 64
    fractions = []
    for T in (2, 4, 8, 16, 32, 64, 128):
        rp, ci = oracle.mask_radial(T, S, 1)     # block 1 = token level
        fractions.append(len(ci) / (T * S * S))
    steps = np.diff(fractions)
    assert np.all(steps > 1.0) and np.all(steps < 4.0)
    assert steps[-3:].max() - steps[-3:].min() < 0.5


def test_radial_long_workload_count():
    """125 frames x 3,600 tokens, 128-token blocks: the count the same reading gives
    when re-derived by a second, independent pair test (minimum in-frame distance
    between the two blocks' token runs, per frame pair)."""
    T, S, block = 125, 3600, 128
    rp, ci = oracle.mask_radial(T, S, block)
    assert len(rp) - 1 == 3516
    assert len(ci) == 2718652
    lens = np.diff(rp)
    assert lens.min() == 412 and lens.max() == 871
    # independent check on a few rows: per (q-frame run, k-frame run) minimum distance
    N = T * S
    rng = np.random.default_rng(0)
    for i in rng.choice(3516, 12, replace=False).tolist() + [3515]:
        got = set(ci[rp[i]:rp[i + 1]].tolist())
        want = set()
        q0, q1 = i * block, min(N, (i + 1) * block)
        for j in range(3516):
            k0, k1 = j * block, min(N, (j + 1) * block)
            ok = False
            for f in range(q0 // S, (q1 - 1) // S + 1):
                qa, qb = max(q0, f * S) - f * S, min(q1, (f + 1) * S) - 1 - f * S
                for g in range(k0 // S, (k1 - 1) // S + 1):
                    ka, kb = max(k0, g * S) - g * S, min(k1, (g + 1) * S) - 1 - g * S
                    d = abs(f - g)
                    gap = max(0, ka - qb, qa - kb)
                    r = d.bit_length() - 1 if d >= 2 else 0
                    if d <= 1 or gap * (1 << r) < S:
                        ok = True
            if ok:
                want.add(j)
        assert got == want, i


# ----------------------------------------------------------------------- NABLA
def test_select_golden(golden_dir):
    with open(os.path.join(golden_dir, "select_hand.json")) as f:
        g = json.load(f)
    for c in g["nabla"]:
        kept, _, _ = oracle.nabla_select_row(np.array(c["p"]), c["thr"])
        assert list(kept) == c["kept"], c
    for c in g["ar"]:
        z = np.array(c["z"], dtype=np.float64)
        forced = np.zeros(len(z), dtype=bool)
        for lo, hi in c["forced"]:
            forced[lo:hi] = True
        kept, _ = oracle.ar_select_row(z, c["topk"], forced)
        assert list(kept) == c["kept"], c


def test_nabla_map_golden(golden_dir):
    """The whole NABLA step on a hand-worked case (pool -> map scaled by 1/sqrt(D) ->
    softmax over each row -> CDF cut): the pooled means exactly, and the CSR at two
    thresholds chosen so that a softmax over the wrong axis, a 1/D scale or no scale each
    keep other blocks."""
    with open(os.path.join(golden_dir, "nabla_hand.json")) as f:
        g = json.load(f)
    D = g["head_dim"]
    assert g["scale"] == D ** -0.5
    qt = np.array(g["q_tokens"], np.float64)
    kt = np.array(g["k_tokens"], np.float64)
    assert np.array_equal(oracle.pool_blocks(qt, g["block_q"]), np.array(g["q_pooled"], np.float64))
    assert np.array_equal(oracle.pool_blocks(kt, g["block_k"]), np.array(g["k_pooled"], np.float64))
    q, k = qt[None, :, None, :], kt[None, :, None, :]          # [B=1, N, heads=1, D]
    for c in g["cases"]:
        rp, ci, flagged, near_tie = oracle.mask_nabla(q, k, g["block_q"], g["block_k"], g["scale"], c["thr"])
        assert rows_of(rp, ci) == c["kept"], c
        assert not flagged.any()
        for mistake in g["plausible_mistakes"].values():   # the case separates the readings
            if isinstance(mistake, dict):
                assert mistake[str(c["thr"])] != c["kept"]


def _random_row(rng, n):
    z = rng.standard_normal(n) * rng.uniform(0.1, 3.0)
    p = np.exp(z - z.max())
    return p / p.sum()


def test_nabla_subset_bruteforce():
    """The kept set is the minimum-cardinality subset whose mass reaches thr, and the
    largest-mass such subset."""
    rng = np.random.default_rng(7)
    for _ in range(60):
        n = int(rng.integers(2, 11))
        p = _random_row(rng, n)
        thr = float(rng.uniform(0.05, 0.99))
        kept, _, _ = oracle.nabla_select_row(p, thr)
        best = None
        for size in range(1, n + 1):
            subsets = [s for s in itertools.combinations(range(n), size) if p[list(s)].sum() >= thr]
            if subsets:
                best = max(subsets, key=lambda s: p[list(s)].sum())
                break
        assert sorted(best) == list(kept)


def test_nabla_threshold_limits_and_minimality():
    rng = np.random.default_rng(8)
    for _ in range(50):
        n = int(rng.integers(1, 200))
        p = _random_row(rng, n)
        kept, _, _ = oracle.nabla_select_row(p, 1.0)
        assert list(kept) == list(range(n))
        kept, _, _ = oracle.nabla_select_row(p, 1e-12)
        assert list(kept) == [int(np.argmax(p))]
        thr = float(rng.uniform(0.1, 0.95))
        kept, _, _ = oracle.nabla_select_row(p, thr)
        assert p[kept].sum() >= thr - 1e-12
        assert p[kept].sum() - p[kept].min() < thr + 1e-12


def test_pooling_ragged_mean():
    x = np.arange(10, dtype=np.float64)[:, None] * np.ones((1, 3))
    pooled = oracle.pool_blocks(x, 4)          # blocks {0..3}, {4..7}, {8, 9}
    assert np.array_equal(pooled[:, 0], [1.5, 5.5, 8.5])


def test_nabla_mask_threshold_one_keeps_all():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 200, 2, 8))
    k = rng.standard_normal((1, 150, 2, 8))
    rp, ci, fl, nt = oracle.mask_nabla(q, k, 16, 32, 8 ** -0.5, 1.0)
    assert len(ci) == 2 * 13 * 5 and not fl.any()


def test_nabla_tiny_workload_density():
    """The fp32 tiny workload (2 heads, 32 blocks of 64) at threshold 0.9 keeps 29 of
    32 blocks in every row (i.i.d. N(0,1) inputs pool to nearly flat maps)."""
    from workloads import gen
    x = {w: gen.make_tensor("tiny", w) for w in ("q", "k")}
    q = oracle.tile_reorder(x["q"].double().numpy(), (8, 16, 16), (4, 4, 4))
    k = oracle.tile_reorder(x["k"].double().numpy(), (8, 16, 16), (4, 4, 4))
    rp, ci, fl, nt = oracle.mask_nabla(q, k, 64, 64, 64 ** -0.5, 0.9)
    assert set(np.diff(rp).tolist()) == {29}


# --------------------------------------------------------------- AR chunk mask
def test_ar_forced_ranges_and_counts():
    forced = oracle.ar_forced_ranges(30 * 52, 21, 1, 3, 64)
    assert forced == [(0, 25), (438, 512)]
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 4680, 2, 16))
    k = rng.standard_normal((1, 32760, 2, 16))
    rp, ci, ties = oracle.mask_ar(q, k, 64, 64, 0.25, 16, forced)
    assert len(rp) - 1 == 2 * 74
    assert set(np.diff(rp).tolist()) == {115}
    keep = oracle.csr_to_bool(rp, ci, 512)
    assert keep[:, :25].all() and keep[:, 438:].all()
    # the 16 selected equal a brute-force ranking of the pooled logits
    qp = oracle.pool_blocks(q[0, :, 1], 64)
    kp = oracle.pool_blocks(k[0, :, 1], 64)
    z = qp @ kp.T * 0.25
    for i in (0, 37, 73):
        ranked = sorted(range(25, 438), key=lambda j: (-z[i, j], j))[:16]
        row = 74 + i
        assert sorted(set(ci[rp[row]:rp[row + 1]].tolist()) - set(range(25)) - set(range(438, 512))) \
            == sorted(ranked)


# --------------------------------------------------------------- composition
def random_csr(rng, n_rows, n_cols, dens):
    keep = rng.random((n_rows, n_cols)) < dens
    return oracle.csr_from_bool(keep), keep


@pytest.mark.parametrize("slabs_a,slabs_b", [(1, 1), (3, 3), (1, 3), (3, 1)])
def test_union_matches_boolean_or(slabs_a, slabs_b):
    """Union = elementwise OR of the dense boolean masks, with a one-slab mask shared."""
    rng = np.random.default_rng(7)
    nq, nk = 9, 13
    (rpa, cia), ka = random_csr(rng, slabs_a * nq, nk, 0.3)
    (rpb, cib), kb = random_csr(rng, slabs_b * nq, nk, 0.4)
    rp, ci = oracle.mask_union(rpa, cia, slabs_a, rpb, cib, slabs_b, nq)
    slabs = max(slabs_a, slabs_b)
    ka = np.tile(ka, (slabs // slabs_a, 1))
    kb = np.tile(kb, (slabs // slabs_b, 1))
    assert np.array_equal(oracle.csr_to_bool(rp, ci, nk), ka | kb)
    assert all(np.all(np.diff(r) > 0) for r in rows_of(rp, ci))   # strictly ascending


def test_union_identities():
    rng = np.random.default_rng(8)
    (rp, ci), keep = random_csr(rng, 12, 20, 0.35)
    empty = oracle.csr_from_bool(np.zeros((12, 20), bool))
    full = oracle.mask_all(12, 20)
    same = oracle.mask_union(rp, ci, 1, rp, ci, 1, 12)
    assert np.array_equal(same[0], rp) and np.array_equal(same[1], ci)
    e = oracle.mask_union(rp, ci, 1, *empty, 1, 12)
    assert np.array_equal(e[0], rp) and np.array_equal(e[1], ci)
    f = oracle.mask_union(rp, ci, 1, *full, 1, 12)
    assert np.array_equal(f[0], full[0]) and np.array_equal(f[1], full[1])
    (rp2, ci2), k2 = random_csr(rng, 12, 20, 0.5)
    ab = oracle.mask_union(rp, ci, 1, rp2, ci2, 1, 12)
    ba = oracle.mask_union(rp2, ci2, 1, rp, ci, 1, 12)
    assert np.array_equal(ab[0], ba[0]) and np.array_equal(ab[1], ba[1])
    # inclusion-exclusion on the counts
    assert ab[0][-1] == keep.sum() + k2.sum() - (keep & k2).sum()


def test_union_rejects_mismatched_slabs():
    rp, ci = oracle.mask_all(2, 3)
    rp2, ci2 = oracle.csr_concat([(rp, ci)] * 2)
    rp3, ci3 = oracle.csr_concat([(rp, ci)] * 3)
    with pytest.raises(ValueError):
        oracle.mask_union(rp2, ci2, 2, rp3, ci3, 3, 2)


def test_sta_heads_per_head_counts_and_order():
    """Each slab equals the shared-window mask of its head; counts follow the closed form."""
    grid, tile = (8, 16, 16), (4, 4, 4)
    windows = [(1, 3, 3), (3, 1, 1), (1, 1, 1), (3, 3, 3)]
    rp, ci = oracle.mask_sta_heads(grid, tile, windows, batch=2)
    n = (8 // 4) * (16 // 4) * (16 // 4)
    assert len(rp) == 2 * len(windows) * n + 1
    for b in range(2):
        for h, win in enumerate(windows):
            s = b * len(windows) + h
            ref_rp, ref_ci = oracle.mask_sta(grid, tile, win)
            lo, hi = rp[s * n], rp[(s + 1) * n]
            assert hi - lo == sta_closed_form_nnz(grid, tile, win)
            assert np.array_equal(rp[s * n:(s + 1) * n + 1] - lo, ref_rp)
            assert np.array_equal(ci[lo:hi], ref_ci)
    # a 1x1x1 window keeps only the diagonal
    s = 2
    lo = rp[s * n]
    assert np.array_equal(ci[lo:lo + n], np.arange(n))


# --------------------------------------------- admissible answers for flagged rows
def test_nabla_cut_admissible():
    """The exact cut is always admissible; one block more or fewer, or a kept block swapped
    for a less probable one, is not, unless the running sum at the cut lies within 1e-5 of
    the threshold (then both neighbouring cuts are)."""
    rng = np.random.default_rng(21)
    for _ in range(200):
        n = int(rng.integers(2, 40))
        p = _random_row(rng, n)
        thr = float(rng.uniform(0.05, 0.99))
        kept, flagged, _ = oracle.nabla_select_row(p, thr)
        assert oracle.nabla_cut_admissible(p, kept, thr)
        order = np.argsort(-p, kind="stable")
        k = len(kept)
        if flagged:
            continue
        assert not oracle.nabla_cut_admissible(p, order[:k - 1], thr) or k == 1
        if k < n:
            assert not oracle.nabla_cut_admissible(p, order[:k + 1], thr)
            gap = p[order[k - 1]] - p[order[k]]
            if gap > 1e-5 * p[order[k - 1]]:            # not a tie: the swap is a different answer
                swapped = np.concatenate([order[:k - 1], order[k:k + 1]])
                assert not oracle.nabla_cut_admissible(p, swapped, thr)
    # running sums exactly on the threshold: both cuts are admissible, a third is not
    p = np.array([0.5, 0.25, 0.125, 0.125])
    assert oracle.nabla_cut_admissible(p, [0, 1], 0.75)
    assert oracle.nabla_cut_admissible(p, [0, 1, 2], 0.75)
    assert not oracle.nabla_cut_admissible(p, [0, 1, 2, 3], 0.75)
    assert not oracle.nabla_cut_admissible(p, [0, 2], 0.6)            # not a prefix
    assert not oracle.nabla_cut_admissible(p, [], 0.6)
    assert oracle.nabla_cut_admissible(p, [0, 1, 2, 3], 1.0)
    assert not oracle.nabla_cut_admissible(p, [0, 1, 2], 1.0)


def test_topk_admissible():
    z = np.array([3.0, 1.0, 4.0, 1.0, 5.0, 9.0, 2.0, 6.0])
    forced = oracle.forced_flags([(0, 1), (7, 8)], len(z))
    kept, _ = oracle.ar_select_row(z, 3, forced)
    assert list(kept) == [0, 2, 4, 5, 7]
    assert oracle.topk_admissible(z, kept, 3, forced)
    assert not oracle.topk_admissible(z, [0, 2, 4, 5], 3, forced)          # a forced block missing
    assert not oracle.topk_admissible(z, [0, 1, 4, 5, 7], 3, forced)       # 1.0 chosen over 4.0
    assert not oracle.topk_admissible(z, [0, 2, 4, 5, 6, 7], 3, forced)    # one too many
    # the 3rd and 4th candidates tie within 1e-5: either one is admissible
    z2 = z.copy()
    z2[6] = 4.0 * (1 - 1e-7)
    assert oracle.topk_admissible(z2, [0, 4, 5, 6, 7], 3, forced)
    assert oracle.topk_admissible(z2, [0, 2, 4, 5, 7], 3, forced)
    rng = np.random.default_rng(22)
    for _ in range(100):
        n = int(rng.integers(5, 60))
        zr = rng.standard_normal(n)
        fr = rng.random(n) < 0.2
        kk = int(rng.integers(1, 5))
        kept, _ = oracle.ar_select_row(zr, kk, fr)
        assert oracle.topk_admissible(zr, kept, kk, fr)

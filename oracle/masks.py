"""Block masks (oracle), as CSR lists of kept key blocks.

CSR convention: row r lists the kept key blocks of query block r in ascending
order; row_ptr[n_rows + 1] holds absolute int32 offsets into col_idx.  For masks
computed per (batch, head), row r = (b * heads + h) * n_qblocks + qblock.

A block is a contiguous run of `block` tokens; the last block of a sequence may be
ragged (fewer tokens).
"""
import numpy as np


# ----------------------------------------------------------------------------- CSR
def csr_from_bool(keep):
    """keep: bool [n_rows, n_cols] -> (row_ptr int32 [n_rows+1], col_idx int32)."""
    keep = np.asarray(keep, dtype=bool)
    counts = keep.sum(axis=1)
    row_ptr = np.zeros(keep.shape[0] + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.nonzero(keep)[1]          # row-major order: ascending within a row
    return row_ptr.astype(np.int32), col_idx.astype(np.int32)


def csr_to_bool(row_ptr, col_idx, n_cols):
    n_rows = len(row_ptr) - 1
    keep = np.zeros((n_rows, n_cols), dtype=bool)
    for r in range(n_rows):
        keep[r, col_idx[row_ptr[r]:row_ptr[r + 1]]] = True
    return keep


def mask_all(n_qblocks, n_kblocks):
    """All-ones mask: every query block keeps every key block (dense attention)."""
    return csr_from_bool(np.ones((n_qblocks, n_kblocks), dtype=bool))


# ----------------------------------------------------------------------------- STA
def mask_sta(grid, tile, window):
    """Sliding tile window over the tile grid.

    Sliding Tile Attention explainer (aibr.jp/archives/60739), sec. 3: each query
    tile attends only to the tiles of a window sliding with it, which exploits the
    3D locality of sec. 1.  Readings taken: the window (wt, wh, ww) counts tiles, is
    odd and centred on the query tile, and is clipped at the grid border (border
    tiles attend fewer tiles); key tile j is kept for query tile i iff
    |i_t - j_t| <= wt//2 and |i_h - j_h| <= wh//2 and |i_w - j_w| <= ww//2.
    Tile index = raster index over the tile grid (the tile-major order of
    tile_reorder).
    """
    T, H, W = grid
    tt, th, tw = tile
    if T % tt or H % th or W % tw:
        raise ValueError("grid not divisible by tile")
    if any(w <= 0 or w % 2 == 0 for w in window):
        raise ValueError("window sizes must be odd and positive")
    NT, NH, NW = T // tt, H // th, W // tw
    i = np.arange(NT * NH * NW)
    ct, ch, cw = i // (NH * NW), (i // NW) % NH, i % NW
    wt, wh, ww = (w // 2 for w in window)
    keep = ((np.abs(ct[:, None] - ct[None, :]) <= wt)
            & (np.abs(ch[:, None] - ch[None, :]) <= wh)
            & (np.abs(cw[:, None] - cw[None, :]) <= ww))
    return csr_from_bool(keep)


def mask_sta_heads(grid, tile, windows, batch=1):
    """STA with one window per head: slab b * heads + h uses windows[h].

    Sliding Tile Attention explainer (aibr.jp/archives/60739), sec. 1: besides 3D
    locality, attention heads specialise, so a window sized per head is the plain
    extension of the shared window of mask_sta.  The slabs are stacked in
    (batch, head) order, the CSR convention of the per-head masks.
    """
    parts = [mask_sta(grid, tile, windows[h]) for h in range(len(windows))]
    rows = [parts[h] for _ in range(batch) for h in range(len(windows))]
    return csr_concat(rows)


def csr_concat(parts):
    """Stack CSR masks (row_ptr, col_idx) vertically."""
    row_ptr, cols, off = [0], [], 0
    for rp, ci in parts:
        row_ptr.extend((np.asarray(rp[1:], np.int64) + off).tolist())
        cols.append(np.asarray(ci, np.int64))
        off += int(rp[-1])
    return (np.asarray(row_ptr, np.int32),
            np.concatenate(cols).astype(np.int32) if cols else np.zeros(0, np.int32))


def mask_union(rp_a, ci_a, slabs_a, rp_b, ci_b, slabs_b, n_qblocks):
    """Row-by-row union of two block masks.

    NABLA explainer (aibr.jp/archives/124678), sec. 2 and 4: the NABLA mask works
    alongside other accelerations and the two combine; reading taken: a combined
    mask keeps a block pair iff either mask keeps it (e.g. NABLA with an STA
    window).  A mask with one slab is shared by every (batch, head) slab of the
    other; the result has max(slabs_a, slabs_b) slabs.
    """
    slabs = max(slabs_a, slabs_b)
    if slabs_a not in (1, slabs) or slabs_b not in (1, slabs):
        raise ValueError("slab counts must be equal or 1")
    rows = []
    for s in range(slabs):
        sa, sb = (s if slabs_a > 1 else 0), (s if slabs_b > 1 else 0)
        for i in range(n_qblocks):
            ra, rb = sa * n_qblocks + i, sb * n_qblocks + i
            a = set(ci_a[rp_a[ra]:rp_a[ra + 1]].tolist())
            b = set(ci_b[rp_b[rb]:rp_b[rb + 1]].tolist())
            rows.append(sorted(a | b))
    row_ptr = np.zeros(len(rows) + 1, np.int64)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col_idx = np.asarray([c for r in rows for c in r], np.int64)
    return row_ptr.astype(np.int32), col_idx.astype(np.int32)


# -------------------------------------------------------------------------- radial
def radial_keep_tokens(fq, sq, fk, sk, S):
    """Token-level radial rule (broadcasts over arrays).

    Radial Attention explainer (aibr.jp/archives/112136), sec. 2-3: attention stays
    dense between nearby frames and the spatial window shrinks exponentially as the
    temporal distance grows (energy decay), which gives O(n log n) kept pairs.
    Reading taken: with d = |fq - fk| and r = floor(log2 d), keep iff d <= 1 or
    |sq - sk| * 2^r < S, i.e. the spatial window halves at each doubling of d.
    Spatial distance = distance of raster in-frame indices s = h * W + w.
    """
    d = np.abs(np.asarray(fq, dtype=np.int64) - np.asarray(fk, dtype=np.int64))
    r = np.frexp(np.maximum(d, 1).astype(np.float64))[1].astype(np.int64) - 1  # floor(log2 d)
    ds = np.abs(np.asarray(sq, dtype=np.int64) - np.asarray(sk, dtype=np.int64))
    return (d <= 1) | (ds * (np.int64(1) << r) < S)


def mask_radial(T, S, block):
    """Block-level radial mask over raster order: N = T*S tokens, blocks of `block`
    tokens (last one ragged); key block J is kept for query block I iff any token
    pair (q in I, k in J) is kept by the token rule (reading: 'any').

    For a run of query tokens with in-frame indices [a, e] in frame f and a key
    frame g at distance d: d <= 1 keeps the whole key frame; otherwise the kept key
    indices are those within w = floor((S - 1) / 2^r) of some s in [a, e] (the
    largest w with w * 2^r < S), i.e. [a - w, e + w] clipped to the frame.  The
    key tokens of that interval touch blocks floor(lo / block) .. floor(hi / block).
    """
    N = T * S
    nb = -(-N // block)
    keep = np.zeros((nb, nb), dtype=bool)
    g = np.arange(T)
    for i in range(nb):
        q0, q1 = i * block, min((i + 1) * block, N)
        for f in range(q0 // S, (q1 - 1) // S + 1):
            a = max(q0, f * S) - f * S
            e = min(q1, (f + 1) * S) - 1 - f * S
            d = np.abs(f - g)
            r = np.array([int(x).bit_length() - 1 if x >= 2 else 0 for x in d])  # floor(log2 d)
            w = (S - 1) >> r
            lo = np.where(d <= 1, 0, np.maximum(0, a - w))
            hi = np.where(d <= 1, S - 1, np.minimum(S - 1, e + w))
            for gg in range(T):
                keep[i, (gg * S + lo[gg]) // block:(gg * S + hi[gg]) // block + 1] = True
    return csr_from_bool(keep)


# --------------------------------------------------------------------------- NABLA
def pool_blocks(x, block):
    """Mean over the valid tokens of each block: x [n, D] fp64 -> [ceil(n/block), D].

    NABLA explainer (aibr.jp/archives/124678), sec. 3: Q and K are downsampled per
    block by average pooling.  Reading: a ragged last block is averaged over its
    valid tokens only."""
    n = x.shape[0]
    nb = -(-n // block)
    return np.stack([x[i * block:min((i + 1) * block, n)].mean(axis=0) for i in range(nb)])


def nabla_select_row(p, thr, tol=1e-5):
    """One row of the NABLA cut.

    NABLA explainer, sec. 3: from the downsampled attention map, a threshold on the
    cumulative distribution decides which blocks are kept (binarisation), per
    sample, adaptively (sec. 1).  Readings taken: sort the row's block
    probabilities in descending order (ties: lower block index first), take running
    sums C_k, keep the shortest prefix whose sum reaches thr (C_k >= thr, the
    crossing block included); thr = 1 keeps every block.

    Returns (kept ascending indices, flagged, near_tie) where `flagged` marks a row
    whose cumulative mass at the cut, or just before it, lies within `tol` of thr,
    and `near_tie` marks a row whose last kept and first dropped probabilities
    differ by less than tol relative (both are places where rounding may flip the
    decision)."""
    n = len(p)
    order = np.argsort(-p, kind="stable")
    ps = p[order]
    c = np.cumsum(ps)
    if thr >= 1.0:
        return np.arange(n), False, False
    k = int(np.searchsorted(c, thr, side="left"))   # first k with c[k] >= thr
    if k >= n:
        k = n - 1
    flagged = abs(c[k] - thr) < tol or (k > 0 and abs(c[k - 1] - thr) < tol)
    near_tie = k + 1 < n and (ps[k] - ps[k + 1]) < tol * ps[k]
    return np.sort(order[:k + 1]), bool(flagged), bool(near_tie)


def _pooled_logits(qh, kh, block_q, block_k, scale):
    """Z = pool(Q) pool(K)^T * scale for one (batch, head); fp64."""
    return (pool_blocks(qh, block_q) @ pool_blocks(kh, block_k).T) * scale


def pooled_maps(q, k, block_q, block_k, scale, softmax):
    """The pooled map of every (batch, head), in (b, h) order: Z = pool(Q) pool(K)^T *
    scale, or with softmax=True its row softmax p (one distribution over the key blocks
    per query block).  NABLA explainer (aibr.jp/archives/124678), sec. 3."""
    B, _, Hh, _ = q.shape
    for b in range(B):
        for h in range(Hh):
            z = _pooled_logits(np.asarray(q[b, :, h, :], np.float64),
                               np.asarray(k[b, :, h, :], np.float64), block_q, block_k, scale)
            if softmax:
                p = np.exp(z - z.max(axis=1, keepdims=True))
                z = p / p.sum(axis=1, keepdims=True)
            yield z


def mask_nabla(q, k, block_q, block_k, scale, thr):
    """NABLA mask per (batch, head).

    NABLA explainer (aibr.jp/archives/124678), sec. 3: mean-pool Q and K per block,
    compute a small full attention map from the pooled vectors, turn each row into
    a distribution (softmax), and binarise it with the CDF threshold.  Reading: the
    map uses the attention's own scale (1/sqrt(D) in every workload).

    q: [B, Nq, Hh, D], k: [B, Nk, Hh, D] (fp64 or anything numpy upcasts).
    Returns (row_ptr, col_idx, flagged bool[rows], near_tie bool[rows]) with rows
    ordered (b, h, qblock)."""
    nbk = -(-k.shape[1] // block_k)
    keeps, flags, ties = [], [], []
    for p in pooled_maps(q, k, block_q, block_k, scale, softmax=True):
        for row in p:
            kept, fl, nt = nabla_select_row(row, thr)
            m = np.zeros(nbk, dtype=bool)
            m[kept] = True
            keeps.append(m)
            flags.append(fl)
            ties.append(nt)
    rp, ci = csr_from_bool(np.array(keeps))
    return rp, ci, np.array(flags), np.array(ties)


def nabla_cut_admissible(p, kept, thr, tol=1e-5):
    """Whether `kept` (block indices) is a cut that rounding of the running sums could
    give for probabilities p at threshold thr: its mass reaches thr - tol, dropping its
    smallest block leaves less than thr + tol (minimal), and it is a descending prefix up
    to ties (no dropped block is more probable than a kept one by more than tol
    relative).  For a row whose running sum at the cut lies within tol of thr (a flagged
    row) both neighbouring cuts pass; far from the threshold only the exact cut does."""
    p = np.asarray(p, np.float64)
    kept = np.asarray(kept, np.int64)
    if thr >= 1.0:
        return len(kept) == len(p)
    if len(kept) == 0 or len(np.unique(kept)) != len(kept):
        return False
    inside = np.zeros(len(p), bool)
    inside[kept] = True
    mass, smallest = p[inside].sum(), p[inside].min()
    if mass < thr - tol or mass - smallest >= thr + tol:
        return False
    return bool(inside.all() or smallest >= p[~inside].max() * (1.0 - tol))


# ---------------------------------------------------------- autoregressive chunk mask
def ar_forced_ranges(frame_tokens, n_frames, anchor_frames, recent_frames, block):
    """[lo, hi) key-block ranges always kept for an autoregressive chunk step.

    Sparse Forcing summary (gist.science/ja/paper/2604.21221), part 2: who is in the
    scene and where (the first frames) are kept as a persistent anchor memory, and
    the most recent frames are looked at closely.  Readings: anchors = every key
    block holding a token of the first `anchor_frames` frames; recent = every key
    block holding a token of the last `recent_frames` frames of the cache."""
    nk = frame_tokens * n_frames
    nbk = -(-nk // block)
    anchor_end = anchor_frames * frame_tokens             # tokens [0, anchor_end)
    recent_start = (n_frames - recent_frames) * frame_tokens
    return [(0, -(-anchor_end // block)), (recent_start // block, nbk)]


def ar_select_row(z, topk, is_forced):
    """One row of the anchor + recent + top-k selection (see mask_ar).

    Returns (kept ascending indices, near_tie)."""
    cand = np.nonzero(~is_forced)[0]
    order = cand[np.argsort(-z[cand], kind="stable")]
    m = is_forced.copy()
    m[order[:topk]] = True
    tie = False
    if 0 < topk < len(order):
        za, zb = z[order[topk - 1]], z[order[topk]]
        tie = bool((za - zb) <= 1e-5 * max(abs(za), 1e-300))
    return np.nonzero(m)[0], tie


def mask_ar(q, k, block_q, block_k, scale, topk, forced):
    """Anchor + recent + top-k mask per (batch, head).

    Sparse Forcing summary, part 2: besides the anchor and recent blocks, only the
    past blocks that are needed are looked at.  Reading: the needed blocks are the
    `topk` non-forced key blocks with the largest pooled logit
    Z = pool(Q) pool(K)^T * scale (ties: lower block index first), chosen per query
    block and per head.

    Returns (row_ptr, col_idx, near_tie bool[rows]); near_tie marks rows whose k-th
    and (k+1)-th selected logits differ by less than 1e-5 relative."""
    nbk = -(-k.shape[1] // block_k)
    is_forced = forced_flags(forced, nbk)
    keeps, ties = [], []
    for z in pooled_maps(q, k, block_q, block_k, scale, softmax=False):
        for row in z:
            kept, tie = ar_select_row(row, topk, is_forced)
            m = np.zeros(nbk, dtype=bool)
            m[kept] = True
            keeps.append(m)
            ties.append(tie)
    rp, ci = csr_from_bool(np.array(keeps))
    return rp, ci, np.array(ties)


def forced_flags(forced, nbk):
    """bool [nbk]: the key blocks inside the forced [lo, hi) ranges."""
    is_forced = np.zeros(nbk, dtype=bool)
    for lo, hi in forced:
        is_forced[lo:hi] = True
    return is_forced


def topk_admissible(z, kept, topk, is_forced, tol=1e-5):
    """Whether `kept` is a selection that rounding of the logits could give: every forced
    block, exactly `topk` others, and no unselected candidate's logit above a selected
    one's by more than tol relative (the k-th / (k+1)-th tie window of mask_ar)."""
    z = np.asarray(z, np.float64)
    kept = np.asarray(kept, np.int64)
    inside = np.zeros(len(z), bool)
    inside[kept] = True
    if len(np.unique(kept)) != len(kept) or not inside[is_forced].all():
        return False
    sel, rest = inside & ~is_forced, ~inside & ~is_forced
    if sel.sum() != min(topk, (~is_forced).sum()):
        return False
    if not rest.any() or not sel.any():
        return True
    lo, hi = z[sel].min(), z[rest].max()
    return bool(hi - lo <= tol * max(abs(lo), 1e-300))

"""KV-cache compaction for chunked autoregressive generation (oracle).

Sparse Forcing summary (gist.science/ja/paper/2604.21221), parts 2-3: the anchor
blocks are kept as persistent memory, the recent ones only where needed, and the
rest of the past is not stored, which cuts the memory to less than half (a 42%
reduction on the page).  Readings taken:
  * what one (batch, head) must keep is the union of the key blocks its mask rows
    keep (anchors, recent blocks and every query block's selected blocks);
  * the compact cache keeps the [batch, tokens, heads, head_dim] layout: the kept
    full blocks of each head are packed from slot 0 in ascending order, and a kept
    ragged last block goes to one shared tail slot after the largest head's full
    blocks, so every compact block has the token count the attention expects;
  * the mask is rewritten onto the compact slots; attention over the compact cache
    then equals attention over the full cache.
"""
import numpy as np


def kv_keep(row_ptr, col_idx, n_slabs, n_qblocks, n_kblocks, nk, block_k):
    """Per slab, the ascending list of key blocks any of its rows keeps, and the
    block -> compact slot map (-1 = dropped).  Returns (keep lists, remap
    [n_slabs, n_kblocks], n_full_max, has_tail)."""
    ragged = nk % block_k != 0
    tail = n_kblocks - 1 if ragged else -1
    keeps = []
    for s in range(n_slabs):
        lo, hi = row_ptr[s * n_qblocks], row_ptr[(s + 1) * n_qblocks]
        keeps.append(np.unique(np.asarray(col_idx[lo:hi], np.int64)))
    n_full = [int(np.sum(k != tail)) for k in keeps]
    n_full_max = max(n_full) if n_full else 0
    remap = np.full((n_slabs, n_kblocks), -1, np.int64)
    for s, k in enumerate(keeps):
        full = k[k != tail]
        remap[s, full] = np.arange(len(full))
        if tail >= 0 and np.any(k == tail):
            remap[s, tail] = n_full_max
    has_tail = bool(tail >= 0 and any(np.any(k == tail) for k in keeps))
    return keeps, remap, n_full_max, has_tail


def compact_tokens(n_full_max, has_tail, nk, block_k):
    """Token count of the compact cache."""
    return n_full_max * block_k + ((nk - (nk // block_k) * block_k) if has_tail else 0)


def kv_compact(x, remap, heads, block_k, n_out):
    """Gather x [B, nk, H, D] into the compact cache [B, n_out, H, D] by the slot map
    (slab = b * heads + h; slab count 1 = one map for every (b, h)).  Slots no block
    maps to are left zero."""
    x = np.asarray(x)
    B, nk, H, D = x.shape
    out = np.zeros((B, n_out, H, D), dtype=x.dtype)
    for b in range(B):
        for h in range(H):
            s = 0 if remap.shape[0] == 1 else b * heads + h
            for j in np.nonzero(remap[s] >= 0)[0]:
                t0, t1 = j * block_k, min(nk, (j + 1) * block_k)
                c0 = remap[s, j] * block_k
                out[b, c0:c0 + (t1 - t0), h] = x[b, t0:t1, h]
    return out


def mask_remap(row_ptr, col_idx, remap, n_qblocks):
    """The mask rewritten onto compact slots (row r of slab r // n_qblocks); rows stay
    ascending because the slot map is increasing."""
    out = np.empty(int(row_ptr[-1]), np.int64)
    for r in range(len(row_ptr) - 1):
        s = 0 if remap.shape[0] == 1 else r // n_qblocks
        cols = np.asarray(col_idx[row_ptr[r]:row_ptr[r + 1]], np.int64)
        out[row_ptr[r]:row_ptr[r + 1]] = remap[s, cols]
    return np.asarray(row_ptr, np.int32), out.astype(np.int32)

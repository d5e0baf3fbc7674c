"""Exact block-sparse softmax attention (oracle), fp64.

Every page treats full 3D attention (every token against every token, quadratic
cost) as the thing being replaced: Radial Attention explainer (aibr.jp/archives/
112136) sec. 1, Sliding Tile Attention explainer (aibr.jp/archives/60739) sec. 1,
NABLA explainer (aibr.jp/archives/124678) sec. 1; the sparse methods compute the
same attention over the kept blocks only (SPADE summary, gist.science/ja/paper/
2608.03335, "The solution", part 3: head-wise sparse attention).  Reading taken:
for a query token of query block i, the keys are all valid tokens of the kept key
blocks J_i, and

    s_j = q . k_j * scale,  m = max_j s_j,  p_j = exp(s_j - m),  l = sum_j p_j,
    o = sum_j p_j v_j / l,  lse = m + ln l.

A row with no kept block has o = 0 and lse = -inf.
"""
import numpy as np


def block_softmax(qi, kj, scale):
    """Softmax probabilities of a query block over a key set: [nq, nk] fp64."""
    s = (qi @ kj.T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return p / p.sum(axis=1, keepdims=True)


def _slab(n_slabs, b, h, heads):
    return 0 if n_slabs == 1 else b * heads + h


def _key_tokens(cols, block_k, nk):
    """Ascending token indices of the kept key blocks."""
    if len(cols) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(j * block_k, min((j + 1) * block_k, nk)) for j in cols])


def attention(q, k, v, row_ptr, col_idx, block_q, block_k, scale, n_slabs=1):
    """q [B, Nq, Hh, D], k/v [B, Nk, Hh, D] -> (o [B, Nq, Hh, D] fp64, lse [B, Hh, Nq] fp64).

    CSR row r = slab * n_qblocks + qblock, slab = 0 when n_slabs == 1, else b*Hh + h."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, nq, Hh, D = q.shape
    nk = k.shape[1]
    nbq = -(-nq // block_q)
    o = np.zeros((B, nq, Hh, D))
    lse = np.full((B, Hh, nq), -np.inf)
    for b in range(B):
        for h in range(Hh):
            base = _slab(n_slabs, b, h, Hh) * nbq
            for i in range(nbq):
                r = base + i
                toks = _key_tokens(col_idx[row_ptr[r]:row_ptr[r + 1]], block_k, nk)
                q0, q1 = i * block_q, min((i + 1) * block_q, nq)
                if len(toks) == 0:
                    continue
                s = (q[b, q0:q1, h] @ k[b, toks, h].T) * scale
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                l = p.sum(axis=1, keepdims=True)
                o[b, q0:q1, h] = (p @ v[b, toks, h]) / l
                lse[b, h, q0:q1] = (m + np.log(l))[:, 0]
    return o, lse


def attention_rows(q_rows, row_tokens, kh, vh, row_ptr, col_idx, row_base,
                   block_q, block_k, scale, chunk=32):
    """Selected output rows of one (batch, head), by the masked-dense definition.

    q_rows [R, D] are the query vectors of query tokens `row_tokens`; kh, vh [Nk, D]
    the head's keys and values; the CSR row of token t is row_base + t // block_q.
    Scores of keys outside the kept blocks are set to -inf, then an ordinary
    softmax over all Nk keys is taken.  Returns (o [R, D], lse [R])."""
    q_rows = np.asarray(q_rows, np.float64)
    nk = kh.shape[0]
    out = np.zeros_like(q_rows)
    lse = np.full(len(q_rows), -np.inf)
    for c0 in range(0, len(q_rows), chunk):
        c1 = min(len(q_rows), c0 + chunk)
        s = (q_rows[c0:c1] @ kh.T) * scale
        allowed = np.zeros((c1 - c0, nk), dtype=bool)
        for a, t in enumerate(row_tokens[c0:c1]):
            r = row_base + int(t) // block_q
            for j in col_idx[row_ptr[r]:row_ptr[r + 1]]:
                allowed[a, j * block_k:min((j + 1) * block_k, nk)] = True
        s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        ok = np.isfinite(m[:, 0])
        m = np.where(np.isfinite(m), m, 0.0)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        with np.errstate(invalid="ignore", divide="ignore"):
            out[c0:c1] = np.where(ok[:, None], (p @ vh) / l, 0.0)
            lse[c0:c1] = np.where(ok, (m + np.log(l))[:, 0], -np.inf)
    return out, lse


def attention_bwd(q, k, v, dout, row_ptr, col_idx, block_q, block_k, scale, n_slabs=1):
    """Gradients of L = sum(dout * o) for o = attention(q, k, v) over the kept blocks:
    returns (dq, dk, dv) fp64 with the shapes of q, k, v.

    The pages report that the sparse patterns also train (Radial Attention explainer,
    sec. 4: faster training as well as inference; Sparse Forcing summary, part 2: the
    model learns the sparse memory), so the path has a backward pass.  Reading taken:
    the gradient of the same exact attention, evaluated by the chain rule step by
    step for each query block i with key set J_i (no saved state):

        s = q K^T * scale, p = softmax(s)          (rows of the block)
        dv_J += p^T dout,  dp = dout V^T
        ds = p * (dp - sum_j p_j dp_j)             (the softmax Jacobian applied to dp)
        dq = ds K * scale, dk_J += ds^T q * scale

    Rows with no kept block contribute nothing."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dout = np.asarray(dout, np.float64)
    B, nq, Hh, D = q.shape
    nk = k.shape[1]
    nbq = -(-nq // block_q)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(Hh):
            base = _slab(n_slabs, b, h, Hh) * nbq
            for i in range(nbq):
                r = base + i
                toks = _key_tokens(col_idx[row_ptr[r]:row_ptr[r + 1]], block_k, nk)
                if len(toks) == 0:
                    continue
                q0, q1 = i * block_q, min((i + 1) * block_q, nq)
                qi, di = q[b, q0:q1, h], dout[b, q0:q1, h]
                kj, vj = k[b, toks, h], v[b, toks, h]
                p = block_softmax(qi, kj, scale)
                dv[b, toks, h] += p.T @ di
                dp = di @ vj.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, q0:q1, h] = ds @ kj * scale
                dk[b, toks, h] += ds.T @ qi * scale
    return dq, dk, dv


def attention_bwd_query_rows(q_rows, row_tokens, dout_rows, kh, vh, row_ptr, col_idx, row_base, block_q, block_k,
                             scale):
    """dq of selected query rows of one (batch, head), by the same steps as attention_bwd.

    q_rows, dout_rows [n, D]; row_tokens [n] = their query positions; kh, vh [Nk, D].
    The CSR row of position t is row_base + t // block_q."""
    nk = kh.shape[0]
    out = np.zeros((len(row_tokens), kh.shape[1]))
    for n, t in enumerate(row_tokens):
        r = row_base + t // block_q
        toks = _key_tokens(col_idx[row_ptr[r]:row_ptr[r + 1]], block_k, nk)
        if len(toks) == 0:
            continue
        kj, vj = kh[toks], vh[toks]
        p = block_softmax(q_rows[n][None], kj, scale)[0]
        dp = vj @ dout_rows[n]
        ds = p * (dp - (p * dp).sum())
        out[n] = ds @ kj * scale
    return out


def attention_bwd_key_block(j, qh, kh, vh, douth, row_ptr, col_idx, row_base, n_qblocks, block_q, block_k, scale):
    """(dk, dv) of the tokens of key block j of one (batch, head): the sums of attention_bwd
    over every query block whose row keeps j.  qh, douth [Nq, D]; kh, vh [Nk, D]."""
    nq, nk = qh.shape[0], kh.shape[0]
    j0, j1 = j * block_k, min((j + 1) * block_k, nk)
    dk = np.zeros((j1 - j0, kh.shape[1]))
    dv = np.zeros_like(dk)
    for i in range(n_qblocks):
        r = row_base + i
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        if j not in set(np.asarray(cols).tolist()):
            continue
        toks = _key_tokens(cols, block_k, nk)
        q0, q1 = i * block_q, min((i + 1) * block_q, nq)
        qi, di = qh[q0:q1], douth[q0:q1]
        p = block_softmax(qi, kh[toks], scale)
        dp = di @ vh[toks].T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        sel = (toks >= j0) & (toks < j1)
        dv += p[:, sel].T @ di
        dk += ds[:, sel].T @ qi * scale
    return dk, dv

"""Pins of the oracle's attention backward (CPU only).

The chain-rule gradients are checked against (1) central finite differences of
L = sum(dout * o) computed with the oracle's forward, (2) torch autograd through
dense fp64 attention with an additive -inf block mask, and (3) invariants of the
softmax gradient: every row of ds sums to zero, so the key gradients of a head
sum to zero and dq ignores a common shift of all keys, while the value gradients
of a head sum to the sum of the output gradients of its non-empty rows."""
import numpy as np
import pytest
import torch

import oracle


def problem(seed, B=1, H=2, D=4, nq=6, nk=7, bq=3, bk=2, dens=0.6, slabs=2, empty_row=True):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, n, H, D)) for n in (nq, nk, nk))
    dout = rng.standard_normal((B, nq, H, D))
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    keep = rng.random((slabs * nbq, nbk)) < dens
    keep[np.arange(slabs * nbq), rng.integers(0, nbk, slabs * nbq)] = True
    if empty_row:
        keep[1] = False
    rp, ci = oracle.csr_from_bool(keep)
    return q, k, v, dout, rp, ci, bq, bk, slabs, keep


def test_finite_differences():
    q, k, v, dout, rp, ci, bq, bk, slabs, _ = problem(1)
    scale = 0.7
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, rp, ci, bq, bk, scale, slabs)
    loss = lambda q_, k_, v_: float((oracle.attention(q_, k_, v_, rp, ci, bq, bk, scale, slabs)[0] * dout).sum())
    eps = 1e-6
    for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.allclose(g, num, rtol=1e-6, atol=1e-8), which


def test_matches_torch_autograd_dense_masked():
    q, k, v, dout, rp, ci, bq, bk, slabs, keep = problem(2, B=2, H=3, D=8, nq=40, nk=33, bq=8, bk=5,
                                                         slabs=6, empty_row=False)
    scale = 0.35
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, rp, ci, bq, bk, scale, slabs)
    B, nq, H, D = q.shape
    nk = k.shape[1]
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), requires_grad=True) for x in (q, k, v))
    bias = torch.zeros(B, H, nq, nk, dtype=torch.float64)
    for b in range(B):
        for h in range(H):
            m = keep[(b * H + h) * (-(-nq // bq)):(b * H + h + 1) * (-(-nq // bq))]
            tokmask = np.repeat(np.repeat(m, bq, axis=0)[:nq], bk, axis=1)[:, :nk]
            bias[b, h][torch.from_numpy(~tokmask)] = -np.inf
    att = torch.softmax(tq @ tk.transpose(-1, -2) * scale + bias, dim=-1)
    o = att @ tv
    o.backward(torch.tensor(dout.transpose(0, 2, 1, 3)))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.allclose(mine, t.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-12)


def test_invariants():
    q, k, v, dout, rp, ci, bq, bk, slabs, keep = problem(3, B=1, H=2, D=6, nq=30, nk=25, bq=6, bk=5, slabs=2)
    scale = 0.5
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, rp, ci, bq, bk, scale, slabs)
    assert np.allclose(dk.sum(axis=1), 0.0, atol=1e-10)
    nbq = -(-30 // bq)
    for h in range(2):
        rows = keep[h * nbq:(h + 1) * nbq].any(axis=1)
        live = np.repeat(rows, bq)[:30]
        assert np.allclose(dv[0, :, h].sum(axis=0), dout[0, live, h].sum(axis=0), atol=1e-10)
    c = np.random.default_rng(9).standard_normal((1, 1, 2, 6))
    dq2, _, _ = oracle.attention_bwd(q, k + c, v, dout, rp, ci, bq, bk, scale, slabs)
    assert np.allclose(dq2, dq, atol=1e-10)
    assert np.all(dq[0, 6:12, 0] == 0)                  # query block 1 of head 0 keeps nothing


def test_sampled_rows_and_key_blocks_match_full():
    q, k, v, dout, rp, ci, bq, bk, slabs, _ = problem(4, B=1, H=2, D=8, nq=40, nk=33, bq=8, bk=5, slabs=2)
    scale = 0.4
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, rp, ci, bq, bk, scale, slabs)
    nbq = 5
    for h in range(2):
        rows = np.array([0, 7, 8, 15, 39])
        got = oracle.attention_bwd_query_rows(q[0, rows, h], rows, dout[0, rows, h], k[0, :, h], v[0, :, h],
                                              rp, ci, h * nbq, bq, bk, scale)
        assert np.allclose(got, dq[0, rows, h], atol=1e-12)
        for j in range(7):
            gk, gv = oracle.attention_bwd_key_block(j, q[0, :, h], k[0, :, h], v[0, :, h], dout[0, :, h], rp, ci,
                                                    h * nbq, nbq, bq, bk, scale)
            assert np.allclose(gk, dk[0, 5 * j:min(33, 5 * j + 5), h], atol=1e-12)
            assert np.allclose(gv, dv[0, 5 * j:min(33, 5 * j + 5), h], atol=1e-12)

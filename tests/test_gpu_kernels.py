"""GPU parity of each library call on small synthetic problems (all rows compared).

Every case goes through the C ABI (via the ctypes binding) and is compared with
the fp64 oracle on the same inputs: masks and reorders bit-exactly, attention to
the bf16 tolerance (max-abs 2e-2, mean-abs 2e-3) or 1e-4 for fp32."""
import numpy as np
import pytest
import torch

import block_sparse_attention_masks_amd as vsa
import oracle
from mask_parity import check_nabla, check_topk

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16_MAX, BF16_MEAN, F32_MAX = 2e-2, 2e-3, 1e-4


def to_np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def csr_np(rp, ci):
    rp = rp.cpu().numpy()
    return rp, ci[: int(rp[-1])].cpu().numpy()


def rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float64) * scale).to(dtype)


# --------------------------------------------------------------------- reorder
@pytest.mark.parametrize("grid,tile,heads,dim,dtype", [
    ((8, 16, 16), (4, 4, 4), 2, 64, torch.float32),
    ((6, 16, 24), (6, 8, 8), 3, 128, torch.bfloat16),
    ((4, 8, 16), (1, 8, 8), 5, 128, torch.bfloat16),
    ((3, 5, 7), (1, 1, 7), 1, 8, torch.bfloat16),      # 16-byte rows
])
def test_tile_reorder_bit_exact(grid, tile, heads, dim, dtype):
    n = int(np.prod(grid))
    x = rand((2, n, heads, dim), dtype, 1)
    y = vsa.vsa_tile_reorder(x.to(DEV), grid, tile)
    want = oracle.tile_reorder(x.numpy() if dtype == torch.float32 else x.view(torch.int16).numpy(), grid, tile)
    got = y.cpu()
    got = got.numpy() if dtype == torch.float32 else got.view(torch.int16).numpy()
    assert np.array_equal(got, want)
    back = vsa.vsa_tile_reorder(y, grid, tile, inverse=True)
    assert torch.equal(back.cpu(), x)


# ----------------------------------------------------------------------- masks
@pytest.mark.parametrize("grid,tile,window", [
    ((8, 16, 16), (4, 4, 4), (1, 3, 3)), ((30, 48, 80), (6, 8, 8), (3, 3, 5)),
    ((1, 3, 3), (1, 1, 1), (1, 3, 3)), ((12, 12, 12), (2, 2, 2), (5, 3, 7)),
    ((8, 16, 16), (4, 4, 4), (3, 7, 7)), ((2, 2, 2), (2, 2, 2), (1, 1, 1)),
])
def test_mask_sta_bit_exact(grid, tile, window):
    rp, ci = csr_np(*vsa.vsa_mask_sta(grid, tile, window, DEV))
    orp, oci = oracle.mask_sta(grid, tile, window)
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci)


@pytest.mark.parametrize("T,S,block", [(5, 8, 2), (3, 10, 4), (9, 7, 5), (12, 16, 8), (6, 5, 13),
                                       (17, 4, 3), (1, 9, 4), (16, 20, 32), (40, 300, 64),
                                       (33, 1000, 128), (2, 100, 7)])
def test_mask_radial_bit_exact(T, S, block):
    rp, ci = csr_np(*vsa.vsa_mask_radial(T, S, block, DEV))
    orp, oci = oracle.mask_radial(T, S, block)
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci)


@pytest.mark.parametrize("grid,tile,windows,batch", [
    ((8, 16, 16), (4, 4, 4), [(1, 3, 3), (3, 1, 1), (1, 1, 1), (3, 3, 3)], 2),
    ((30, 48, 80), (6, 8, 8), [(3, 3, 5), (1, 3, 3), (5, 5, 9)], 1),
    ((12, 12, 12), (2, 2, 2), [(13, 13, 13), (3, 5, 7)], 3),           # a window wider than the grid
])
def test_mask_sta_heads_bit_exact(grid, tile, windows, batch):
    rp, ci = csr_np(*vsa.vsa_mask_sta_heads(grid, tile, windows, DEV, batch=batch))
    orp, oci = oracle.mask_sta_heads(grid, tile, windows, batch)
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci)


@pytest.mark.parametrize("nq,nk,slabs_a,slabs_b,da,db", [
    (9, 13, 1, 1, 0.3, 0.4), (20, 300, 3, 3, 0.5, 0.2),      # rows longer than a wave
    (16, 40, 1, 4, 0.1, 0.6), (16, 40, 4, 1, 0.6, 0.0),      # shared one-slab masks; an empty mask
    (7, 2000, 2, 2, 0.9, 0.9),                                # long, mostly overlapping rows
])
def test_mask_union_bit_exact(nq, nk, slabs_a, slabs_b, da, db):
    rng = np.random.default_rng(nq * 1000 + nk)
    ka = rng.random((slabs_a * nq, nk)) < da
    kb = rng.random((slabs_b * nq, nk)) < db
    ka[0] = False                                             # an empty row in A
    rpa, cia = oracle.csr_from_bool(ka)
    rpb, cib = oracle.csr_from_bool(kb)
    dev = lambda x: torch.from_numpy(np.concatenate([x, np.zeros(1, np.int32)]) if len(x) == 0 else x).to(DEV)
    rp, ci = csr_np(*vsa.vsa_mask_union(dev(rpa), dev(cia), slabs_a, dev(rpb), dev(cib), slabs_b, nq, nk))
    orp, oci = oracle.mask_union(rpa, cia, slabs_a, rpb, cib, slabs_b, nq)
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci)


@pytest.mark.parametrize("nq,nk,bq,bk,thr,dtype", [
    (2048, 2048, 64, 64, 0.9, torch.float32), (1000, 777, 64, 32, 0.5, torch.bfloat16),
    (300, 4100, 50, 16, 0.95, torch.bfloat16), (129, 129, 128, 1, 0.7, torch.float32),
    (500, 500, 64, 64, 1.0, torch.bfloat16),
    # rows longer than 1,024 and 2,048 blocks: 8 and 16 sort slots per thread
    (130, 1500, 64, 1, 0.7, torch.bfloat16), (70, 4096, 64, 1, 0.5, torch.float32),
])
def test_mask_nabla_bit_exact(nq, nk, bq, bk, thr, dtype):
    q = rand((1, nq, 3, 128), dtype, 2, 1.0)
    k = rand((1, nk, 3, 128), dtype, 3, 1.0)
    q[..., :8] += 2.0 * torch.linspace(-1, 1, nq).reshape(1, nq, 1, 1).to(dtype)   # some structure
    k[..., :8] += 2.0 * torch.linspace(-1, 1, nk).reshape(1, nk, 1, 1).to(dtype)
    scale = 128 ** -0.5
    rp, ci = csr_np(*vsa.vsa_mask_nabla(q.to(DEV), k.to(DEV), bq, bk, scale, threshold=thr))
    print(f"nabla mask {nq}x{nk} blocks {bq}/{bk} thr {thr}: {check_nabla(rp, ci, to_np(q), to_np(k), bq, bk, scale, thr)}")


def test_mask_nabla_two_batches_bit_exact():
    """Two batches of five heads, ragged last blocks on both sides: the pooled means of every
    (batch, block, head) reach the score of their own (batch, head) slab."""
    q = rand((2, 600, 5, 128), torch.bfloat16, 12, 1.0)
    k = rand((2, 1000, 5, 128), torch.bfloat16, 13, 1.0)
    q[..., :8] += 2.0 * torch.linspace(-1, 1, 600).reshape(1, 600, 1, 1).to(q.dtype)
    k[..., :8] += 2.0 * torch.linspace(-1, 1, 1000).reshape(1, 1000, 1, 1).to(k.dtype)
    q[1] *= -1.0   # the second batch keeps other blocks than the first
    scale = 128 ** -0.5
    rp, ci = csr_np(*vsa.vsa_mask_nabla(q.to(DEV), k.to(DEV), 64, 64, scale, threshold=0.8))
    print(f"nabla mask 2 batches: {check_nabla(rp, ci, to_np(q), to_np(k), 64, 64, scale, 0.8)}")


@pytest.mark.parametrize("nk,bk,forced,topk", [
    (3000, 64, [(0, 5), (40, 47)], 6),
    (2000, 1, [(0, 25), (1900, 2000)], 16),     # 2,000 key blocks: 8 sort slots per thread
    (300, 64, [(0, 1)], 16),                    # fewer blocks than forced + k (5, ragged last): keep all
])
def test_mask_topk_forced_bit_exact(nk, bk, forced, topk):
    q = rand((2, 700, 2, 128), torch.bfloat16, 4)
    k = rand((2, nk, 2, 128), torch.bfloat16, 5)
    rp, ci = csr_np(*vsa.vsa_mask_nabla(q.to(DEV), k.to(DEV), 64, bk, 0.1, topk=topk, forced=forced))
    counts, _ = check_topk(rp, ci, to_np(q), to_np(k), 64, bk, 0.1, topk, forced)
    print(f"top-k mask nk {nk} block {bk}: {counts}")
    assert set(np.diff(rp).tolist()) == {min(-(-nk // bk), sum(hi - lo for lo, hi in forced) + topk)}


# ------------------------------------------------------------------- attention
def _check(o_gpu, lse_gpu, o_ref, lse_ref, dtype):
    o = to_np(o_gpu)
    err = np.abs(o - o_ref)
    if dtype == torch.float32:
        assert err.max() <= F32_MAX, err.max()
    else:
        assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (err.max(), err.mean())
    lse = lse_gpu.cpu().double().numpy()
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - lse_ref[fin]).max() < (1e-4 if dtype == torch.float32 else 2e-2)


CASES = [
    # nq, nk, heads, D, bq, bk, density, slabs, dtype
    (256, 256, 2, 128, 64, 64, 1.0, 1, torch.bfloat16),
    (1000, 1000, 3, 128, 128, 128, 0.4, 1, torch.bfloat16),
    (777, 1234, 2, 128, 384, 384, 0.6, 2, torch.bfloat16),       # ragged q and k tails
    (500, 900, 2, 64, 100, 70, 0.5, 2, torch.bfloat16),          # blocks not multiples of 64
    (130, 4100, 1, 128, 64, 64, 0.2, 1, torch.bfloat16),         # nq != nk, long keys
    (300, 300, 2, 128, 300, 1, 0.3, 2, torch.bfloat16),          # one-token key blocks
    (1100, 800, 2, 128, 256, 128, 0.5, 2, torch.bfloat16),       # 8-wave workgroups, ragged
    (1600, 1500, 1, 64, 768, 256, 0.7, 1, torch.bfloat16),       # 12-wave, two per block
    (2048, 2048, 2, 64, 64, 64, 0.5, 2, torch.float32),
    (200, 333, 2, 128, 32, 48, 0.5, 1, torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_attention_parity(case):
    nq, nk, H, D, bq, bk, dens, slabs, dtype = case
    scale = D ** -0.5
    q, k, v = rand((1, nq, H, D), dtype, 10), rand((1, nk, H, D), dtype, 11), rand((1, nk, H, D), dtype, 12)
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    rng = np.random.default_rng(13)
    keep = rng.random((slabs * nbq, nbk)) < dens
    keep[np.arange(slabs * nbq), rng.integers(0, nbk, size=slabs * nbq)] = True
    if slabs * nbq > 2:
        keep[1] = False                                           # an empty row
    rp, ci = oracle.csr_from_bool(keep)
    o_ref, lse_ref = oracle.attention(to_np(q), to_np(k), to_np(v), rp, ci, bq, bk, scale, slabs)
    o, lse = vsa.vsa_block_sparse_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV),
                                           torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV),
                                           bq, bk, slabs, scale)
    _check(o, lse, o_ref, lse_ref, dtype)


@pytest.mark.parametrize("B,H,D,nq,nk,bq,bk", [
    (2, 3, 128, 900, 830, 384, 384),   # 12-wave blocks, ragged last key tile
    (2, 3, 64, 900, 830, 64, 64),      # 4-wave key split (KS = 2), head_dim 64
])
def test_packed_v_transpose(B, H, D, nq, nk, bq, bk):
    """A call that neither groups nor splits uses its workspace for V^T alone: after the call it
    holds V as [batch, heads, 64-key tile, head_dim, 64], keys past nk zero, bit for bit.  The
    output matches the oracle and equals the row-major-V run (no workspace) to rounding."""
    slabs = B * H
    scale = D ** -0.5
    q, k, v = rand((B, nq, H, D), torch.bfloat16, 60), rand((B, nk, H, D), torch.bfloat16, 61), \
        rand((B, nk, H, D), torch.bfloat16, 62)
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    rng = np.random.default_rng(63)
    keep = rng.random((slabs * nbq, nbk)) < 0.6
    keep[np.arange(slabs * nbq), rng.integers(0, nbk, size=slabs * nbq)] = True
    keep[:, -1] = True                                            # the ragged last key block
    rp, ci = oracle.csr_from_bool(keep)
    rpd, cid = torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ntile = -(-nk // 64)
    vt_bytes = 2 * B * H * ntile * 64 * D
    assert vsa.attn_fwd_workspace_bytes(qd, kd, rpd, cid, bq, bk, slabs) == vt_bytes   # V^T only
    ws = torch.full((vt_bytes,), 0xff, dtype=torch.uint8, device=DEV)
    o, lse = vsa.vsa_block_sparse_attn_fwd(qd, kd, vd, rpd, cid, bq, bk, slabs, scale, workspace=ws)
    torch.cuda.synchronize()
    want = torch.zeros((B, ntile * 64, H, D), dtype=torch.bfloat16)
    want[:, :nk] = v
    want = want.view(B, ntile, 64, H, D).permute(0, 3, 1, 4, 2).contiguous()   # [B, H, tile, D, 64]
    got = ws.view(torch.bfloat16).view(B, H, ntile, D, 64).cpu()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    o_row, _ = vsa.vsa_block_sparse_attn_fwd(qd, kd, vd, rpd, cid, bq, bk, slabs, scale, grouped=False)
    assert (o.float() - o_row.float()).abs().max() <= BF16_MAX
    errs = []
    for b, h in ((0, 0), (B - 1, H - 1)):
        rows = np.concatenate([np.arange(0, 64), rng.choice(nq, 64, replace=False), [nq - 1]])
        base = (b * H + h) * nbq
        ref, ref_lse = oracle.attention_rows(to_np(q[b, rows, h]), rows, to_np(k[b, :, h]), to_np(v[b, :, h]),
                                             rp, ci, base, bq, bk, scale)
        errs.append(np.abs(o[b, rows, h].cpu().double().numpy() - ref))
        assert np.abs(lse[b, h, rows].cpu().double().numpy() - ref_lse).max() < 2e-2
    err = np.concatenate(errs)
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN


@pytest.mark.parametrize("B,H,D,nq,nk,bq,bk", [
    (1, 48, 128, 2000, 2048, 64, 64),    # the grouped plan (12 waves, 6 blocks per group)
    (1, 2, 128, 900, 830, 384, 384),     # 12-wave blocks, packed V
    (1, 3, 64, 500, 700, 64, 64),        # too few rows for one round: split key streams
])
def test_attention_mask_keeping_nothing(B, H, D, nq, nk, bq, bk):
    """A per-head mask whose rows are all empty (the row pointers all zero, no column
    entries): every output row is 0 with lse = -inf, and the gradients are exactly 0."""
    slabs = B * H
    q, k, v, do = (rand(s_, torch.bfloat16, sd).to(DEV) for s_, sd in
                   (((B, nq, H, D), 70), ((B, nk, H, D), 71), ((B, nk, H, D), 72), ((B, nq, H, D), 73)))
    nbq = -(-nq // bq)
    rpd = torch.zeros(slabs * nbq + 1, dtype=torch.int32, device=DEV)
    cid = torch.zeros(1, dtype=torch.int32, device=DEV)           # room for one entry, none used
    o, lse = vsa.vsa_block_sparse_attn_fwd(q, k, v, rpd, cid, bq, bk, slabs, D ** -0.5)
    dq, dk, dv = vsa.vsa_block_sparse_attn_bwd(q, k, v, o, do, lse, rpd, cid, bq, bk, slabs, D ** -0.5)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(lse == -float("inf"))
    assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)


def test_attention_one_token():
    """One query token and one key token (one ragged block each, mostly padding): the output
    is v itself, lse = q.k * scale, and the gradients follow from P = 1: dq = dk = 0 and
    dv = dout (the oracle's values, to the bf16 bounds)."""
    D = 128
    scale = D ** -0.5
    q, k, v, do = (rand((1, 1, 2, D), torch.bfloat16, s_) for s_ in (80, 81, 82, 83))
    rp, ci = oracle.csr_from_bool(np.ones((2, 1), bool))
    rpd, cid = torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV)
    o, lse = vsa.vsa_block_sparse_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), rpd, cid, 64, 64, 2, scale)
    dq, dk, dv = vsa.vsa_block_sparse_attn_bwd(q.to(DEV), k.to(DEV), v.to(DEV), o, do.to(DEV), lse, rpd, cid,
                                               64, 64, 2, scale)
    o_ref, lse_ref = oracle.attention(to_np(q), to_np(k), to_np(v), rp, ci, 64, 64, scale, 2)
    rq, rk, rv = oracle.attention_bwd(to_np(q), to_np(k), to_np(v), to_np(do), rp, ci, 64, 64, scale, 2)
    assert torch.equal(o.cpu(), v)                                 # softmax of one score is exactly 1
    assert np.abs(lse.cpu().double().numpy() - lse_ref).max() < 2e-2
    assert np.abs(dv.cpu().double().numpy() - rv).max() <= BWD_BF16_MAX * np.abs(rv).max()
    # dq, dk: dS = P (dP - D) with dP = dout . v and D = dout . o = dout . v, the same fp32 sum (|.| ~ 10 here) taken
    # in two orders, so what is left is its rounding (~1e-6 relative), times |k| or |q| and the scale
    assert np.abs(dq.cpu().double().numpy()).max() <= 1e-4 and np.abs(dk.cpu().double().numpy()).max() <= 1e-4
    assert np.abs(o_ref - to_np(v)).max() == 0 and np.abs(rq).max() < 1e-12 and np.abs(rk).max() < 1e-12


def test_attention_widest_token_rows():
    """Token rows at the widest the bf16 kernels address (heads x head_dim x 2 bytes just below
    2^24: 65,535 heads of 128): forward and backward on 100 tokens (a ragged second block),
    4 sampled heads (the last included) against the oracle."""
    H, D, N, blk = 65_535, 128, 100, 64
    assert H * D * 2 < 1 << 24 <= (H + 1) * D * 2
    scale = D ** -0.5
    g = torch.Generator(device=DEV).manual_seed(95)
    q, k, v, do = (torch.randn((1, N, H, D), generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
                   for _ in range(4))
    keep = np.array([[True, False], [True, True]])
    rp, ci = oracle.csr_from_bool(keep)
    rpd, cid = torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV)
    o, lse = vsa.vsa_block_sparse_attn_fwd(q, k, v, rpd, cid, blk, blk, 1, scale)
    dq, dk, dv = vsa.vsa_block_sparse_attn_bwd(q, k, v, o, do, lse, rpd, cid, blk, blk, 1, scale)
    torch.cuda.synchronize()
    for h in (0, 12_345, 40_000, H - 1):
        qh, kh, vh, dh = (to_np(t[:, :, h:h + 1]) for t in (q, k, v, do))
        o_ref, lse_ref = oracle.attention(qh, kh, vh, rp, ci, blk, blk, scale, 1)
        _check(o[:, :, h:h + 1], lse[:, h:h + 1], o_ref, lse_ref, torch.bfloat16)
        refs = oracle.attention_bwd(qh, kh, vh, dh, rp, ci, blk, blk, scale, 1)
        for got, ref in zip((dq, dk, dv), refs):
            err = np.abs(to_np(got[:, :, h:h + 1]) - ref)
            assert err.max() <= BWD_BF16_MAX * np.abs(ref).max() and err.mean() <= BWD_BF16_MEAN * np.abs(ref).mean()


def test_forward_captured_in_hip_graph():
    """Both forward entries (workspace argument; the library's fixed array) captured in a HIP graph
    on a default-priority stream and replayed three times, with other device work and
    synchronisations between replays and the inputs rewritten in place before the last one: each
    replay equals the eager call on the same inputs bit for bit.  Given out, lse and the
    workspace, neither call allocates, synchronises or records a memset, so the graph holds
    kernel launches only (the grouped plan: union lists, V^T packing, attention)."""
    B, H, D, nq, nk, bq, bk = 1, 8, 128, 2000, 2048, 64, 64
    slabs, scale = B * H, D ** -0.5
    q, k, v = (rand((B, n, H, D), torch.bfloat16, sd).to(DEV) for n, sd in ((nq, 110), (nk, 111), (nk, 112)))
    q2 = rand((B, nq, H, D), torch.bfloat16, 113).to(DEV)
    rng = np.random.default_rng(114)
    keep = rng.random((slabs * -(-nq // bq), -(-nk // bk))) < 0.4
    keep[:, 0] = True
    rp, ci = oracle.csr_from_bool(keep)
    rpd, cid = torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV)
    ws = torch.empty(vsa.attn_fwd_workspace_bytes(q, k, rpd, cid, bq, bk, slabs), dtype=torch.uint8, device=DEV)

    def eager():
        o_w, l_w = vsa.vsa_block_sparse_attn_fwd(q, k, v, rpd, cid, bq, bk, slabs, scale, workspace=ws)
        o_s, l_s = vsa.vsa_block_sparse_attn_fwd_static(q, k, v, rpd, cid, bq, bk, torch.empty_like(q),
                                                        torch.empty((B, H, nq), dtype=torch.float32, device=DEV),
                                                        slabs, scale)
        torch.cuda.synchronize()
        return o_w, l_w, o_s, l_s

    ref = eager()          # also resolves the fixed array's address before any capture
    outs = [torch.empty_like(q), torch.empty((B, H, nq), dtype=torch.float32, device=DEV),
            torch.empty_like(q), torch.empty((B, H, nq), dtype=torch.float32, device=DEV)]
    graph, side = torch.cuda.CUDAGraph(), torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=side):
        vsa.vsa_block_sparse_attn_fwd(q, k, v, rpd, cid, bq, bk, slabs, scale, out=outs[0], lse=outs[1],
                                      workspace=ws)
        vsa.vsa_block_sparse_attn_fwd_static(q, k, v, rpd, cid, bq, bk, outs[2], outs[3], slabs, scale)
    for rep in range(3):
        if rep == 2:
            q.copy_(q2)
            ref = eager()
        x = torch.randn(1 << 22, device=DEV)
        _ = (x * 2).sum().item()                       # other work and a synchronisation between replays
        for t in outs:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got, want), rep


def test_calls_on_two_streams_overlap_safely():
    """The entries that take a workspace hold no state of their own: two different problems
    run at the same time on two streams (default priority), forward then backward on each,
    give the same bits as the same calls one after the other."""
    probs = []
    for sd, (H, nq, nk, bq, bk) in enumerate(((6, 2000, 2048, 64, 64), (3, 1500, 1300, 128, 128))):
        q, k, v, do = (rand((1, n, H, 128), torch.bfloat16, 120 + 4 * sd + i).to(DEV)
                       for i, n in enumerate((nq, nk, nk, nq)))
        keep = np.random.default_rng(130 + sd).random((H * -(-nq // bq), -(-nk // bk))) < 0.5
        keep[:, -1] = True
        rp, ci = oracle.csr_from_bool(keep)
        probs.append((q, k, v, do, torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV), bq, bk, H))

    def run(p):
        q, k, v, do, rp, ci, bq, bk, H = p
        o, lse = vsa.vsa_block_sparse_attn_fwd(q, k, v, rp, ci, bq, bk, H, 128 ** -0.5)
        return (o, lse) + vsa.vsa_block_sparse_attn_bwd(q, k, v, o, do, lse, rp, ci, bq, bk, H, 128 ** -0.5)

    seq = [run(p) for p in probs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(2):
        got = [None, None]
        for i, (p, st) in enumerate(zip(probs, streams)):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                got[i] = run(p)
        torch.cuda.synchronize()
        for a, b in zip(got, seq):
            for x, y in zip(a, b):
                assert torch.equal(x, y), rep


def test_attention_deterministic_and_dense_mask():
    q, k, v = (rand((1, 1500, 2, 128), torch.bfloat16, s).to(DEV) for s in (20, 21, 22))
    rp, ci = vsa.all_ones_mask(-(-1500 // 128), -(-1500 // 128), DEV)
    o1, l1 = vsa.vsa_block_sparse_attn_fwd(q, k, v, rp, ci, 128, 128)
    o2, l2 = vsa.vsa_block_sparse_attn_fwd(q, k, v, rp, ci, 128, 128)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(t.double().cpu().permute(0, 2, 1, 3) for t in (q, k, v))).permute(0, 2, 1, 3)
    err = (o1.double().cpu() - ref).abs()
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN


# ------------------------------------------------------------------------ SICS
@pytest.mark.parametrize("B,N,H,D,block,dtype", [
    (1, 1000, 2, 128, 64, torch.bfloat16),      # ragged tail block
    (2, 300, 3, 64, 7, torch.float32),
    (1, 130, 40, 128, 384, torch.bfloat16),     # one short block; 640 vectors per row -> two slices
    (1, 65, 1, 64, 1, torch.bfloat16),          # one-row blocks score 1
    (1, 200, 5, 128, 33, torch.float32),        # fp32 at head_dim 128, ragged tail
])
def test_block_sics_matches_oracle(B, N, H, D, block, dtype):
    x = rand((B, N, H, D), dtype, 31)
    x[:, 3] = 0                                  # zero rows add nothing
    got = vsa.vsa_block_sics(x.to(DEV), block).cpu().numpy()
    want = oracle.block_sics(x.double().numpy(), block)
    assert np.allclose(got, want, rtol=1e-10, atol=1e-10)
    if block == 1:
        assert np.all(np.isclose(got, 1.0, rtol=0, atol=1e-14) | (got == 0.0))


# ------------------------------------------------------------ block mean pool
@pytest.mark.parametrize("B,N,H,D,block,dtype", [
    (1, 1000, 2, 128, 64, torch.bfloat16),      # ragged last block (40 rows)
    (2, 300, 3, 64, 7, torch.float32),          # rows split unevenly over the waves
    (1, 130, 40, 128, 384, torch.bfloat16),     # one short block; 10 vector slices per row
    (1, 65, 1, 64, 1, torch.bfloat16),          # one-row blocks: the row itself
    (1, 5000, 24, 128, 128, torch.bfloat16),    # several passes of 16 rows per wave
])
def test_block_mean_pool_bit_exact(B, N, H, D, block, dtype):
    """The pooling pass of the NABLA mask: exact fp64 sums of bf16 rows, one division, so
    the GPU means equal the oracle's bit for bit (fp32 inputs of this range too)."""
    x = rand((B, N, H, D), dtype, 33)
    got = vsa.vsa_block_mean_pool(x.to(DEV), block).cpu().numpy()
    xn = x.double().numpy()
    # the library writes the means block-major, [B, blocks, heads, D]
    want = np.stack([np.stack([oracle.pool_blocks(xn[b, :, h], block) for h in range(H)], axis=1)
                     for b in range(B)])
    assert got.shape == want.shape and np.array_equal(got, want)


# ------------------------------------------------------------ KV compaction
@pytest.mark.parametrize("B,H,D,nq,nk,bq,bk,slabs,dtype,tail_slabs", [
    (1, 3, 128, 300, 1000, 64, 64, 3, torch.bfloat16, (0, 2)),   # ragged tail kept by two heads
    (2, 2, 64, 200, 1024, 50, 64, 4, torch.bfloat16, None),      # no ragged tail
    (1, 2, 128, 130, 777, 64, 96, 1, torch.float32, (0,)),        # one shared mask
])
def test_kv_compaction_matches_oracle(B, H, D, nq, nk, bq, bk, slabs, dtype, tail_slabs):
    from oracle import kvcache
    rng = np.random.default_rng(nk + bk)
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    keep = rng.random((slabs * nbq, nbk)) < 0.2
    keep[:, 0] = True
    if nk % bk:
        keep[:, -1] = False
        for s in tail_slabs:
            keep[s * nbq, -1] = True
    rp, ci = oracle.csr_from_bool(keep)
    k, v = rand((B, nk, H, D), dtype, 51), rand((B, nk, H, D), dtype, 52)
    q = rand((B, nq, H, D), dtype, 53)
    rpd, cid = torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV)
    slot, info = vsa.vsa_kv_plan(rpd, cid, slabs, nbq, nk, bk)
    _, remap, n_full_max, has_tail = kvcache.kv_keep(rp, ci, slabs, nbq, nbk, nk, bk)
    assert np.array_equal(slot.cpu().numpy(), remap)
    assert info[:2].cpu().tolist() == [n_full_max, int(has_tail)]
    n_out = vsa.compact_tokens(info[:2].cpu().tolist(), nk, bk)
    assert n_out == kvcache.compact_tokens(n_full_max, has_tail, nk, bk) and n_out < nk
    kc = vsa.vsa_kv_gather(k.to(DEV), slot, slabs, bk, n_out, out=torch.zeros((B, n_out, H, D), dtype=dtype, device=DEV))
    want = kvcache.kv_compact(k.numpy() if dtype == torch.float32 else k.view(torch.int16).numpy(), remap, H, bk, n_out)
    got = kc.cpu()
    assert np.array_equal(got.numpy() if dtype == torch.float32 else got.view(torch.int16).numpy(), want)
    cc = vsa.vsa_mask_remap(rpd, cid, slabs, nbq, slot, nbk)
    assert np.array_equal(cc.cpu().numpy(), kvcache.mask_remap(rp, ci, remap, nbq)[1])
    # attention over the compact cache is the same computation, tile for tile (compared on the
    # plain path: with a workspace the plan may split the full cache's longer key range over
    # workgroups and not the compact one's, which changes the rounding only)
    vc = vsa.vsa_kv_gather(v.to(DEV), slot, slabs, bk, n_out)
    o_full, l_full = vsa.vsa_block_sparse_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), rpd, cid, bq, bk, slabs,
                                                   grouped=False)
    o_comp, l_comp = vsa.vsa_block_sparse_attn_fwd(q.to(DEV), kc, vc, rpd, cc, bq, bk, slabs, grouped=False)
    assert torch.equal(o_full, o_comp) and torch.equal(l_full, l_comp)
    o_ws, _ = vsa.vsa_block_sparse_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), rpd, cid, bq, bk, slabs)
    assert (o_ws.float() - o_comp.float()).abs().max() <= (BF16_MAX if dtype == torch.bfloat16 else F32_MAX)


# -------------------------------------------------------------- backward
BWD_CASES = [
    # nq, nk, heads, D, bq, bk, density, slabs, dtype
    (256, 256, 2, 128, 64, 64, 1.0, 1, torch.bfloat16),          # dense; key split in both kernels
    (1000, 937, 3, 128, 128, 128, 0.4, 3, torch.bfloat16),       # ragged tails
    (777, 1234, 2, 128, 384, 384, 0.6, 2, torch.bfloat16),       # large blocks, several tiles per block
    (500, 900, 2, 64, 100, 70, 0.5, 2, torch.bfloat16),          # D = 64, blocks not multiples of 64
    (130, 700, 1, 128, 64, 48, 0.3, 1, torch.bfloat16),          # nq != nk
    (300, 300, 2, 64, 64, 64, 0.5, 2, torch.float32),
    (200, 333, 2, 128, 32, 48, 0.5, 1, torch.float32),
    # grouped dK, dV (>= 512 groups): 2 key blocks of 64 per workgroup, per-head masks,
    # a ragged last block alone in the last group; 4 blocks of 32 keys, shared mask
    (128, 4150, 16, 64, 64, 64, 0.5, 16, torch.bfloat16),
    (128, 2070, 32, 128, 64, 32, 0.5, 1, torch.bfloat16),
    # many ragged 64-row query blocks with per-head masks (the key side too few to
    # group); 128-row blocks on both sides
    (4150, 256, 16, 64, 64, 64, 0.5, 16, torch.bfloat16),
    (2100, 2100, 32, 128, 128, 128, 0.4, 1, torch.bfloat16),
]
# Normalised error bounds: |g - ref| over the reference's max (and mean) magnitude.  bf16:
# P and dS are rounded to bf16 before the products (relative 2^-9 each) and D = sum dO * O
# uses the forward's bf16 output, so each summed term carries ~2^-9 = 1.95e-3 relative
# error; the mean error is ~2^-9 of the mean magnitude and no element may exceed 8x that
# of the largest.  fp32: the same sums in fp32 (~1e-6 measured).
BWD_BF16_MAX, BWD_BF16_MEAN, BWD_F32_MAX = 8 * 2.0 ** -9, 2 * 2.0 ** -9, 1e-5


@pytest.mark.parametrize("case", BWD_CASES, ids=[str(i) for i in range(len(BWD_CASES))])
def test_attention_backward_parity(case):
    nq, nk, H, D, bq, bk, dens, slabs, dtype = case
    scale = D ** -0.5
    q, k, v = rand((1, nq, H, D), dtype, 60), rand((1, nk, H, D), dtype, 61), rand((1, nk, H, D), dtype, 62)
    do = rand((1, nq, H, D), dtype, 63)
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    rng = np.random.default_rng(64)
    keep = rng.random((slabs * nbq, nbk)) < dens
    keep[np.arange(slabs * nbq), rng.integers(0, nbk, size=slabs * nbq)] = True
    if slabs * nbq > 2:
        keep[1] = False                                           # an empty row
    rp, ci = oracle.csr_from_bool(keep)
    rpd, cid = torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = vsa.vsa_block_sparse_attn_fwd(qd, kd, vd, rpd, cid, bq, bk, slabs, scale)
    dq, dk, dv = vsa.vsa_block_sparse_attn_bwd(qd, kd, vd, o, dod, lse, rpd, cid, bq, bk, slabs, scale)
    rq, rk, rv = oracle.attention_bwd(to_np(q), to_np(k), to_np(v), to_np(do), rp, ci, bq, bk, scale, slabs)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g = got.cpu().double().numpy()
        err = np.abs(g - ref)
        mx, mn = err.max() / np.abs(ref).max(), err.mean() / np.abs(ref).mean()
        print(f"bwd case {case[:8]} {name}: max_norm {mx:.2e} mean_norm {mn:.2e}", flush=True)
        if dtype == torch.float32:
            assert mx <= BWD_F32_MAX, name
        else:
            assert mx <= BWD_BF16_MAX and mn <= BWD_BF16_MEAN, name
    # rows of the empty query block get exactly zero dq
    if slabs * nbq > 2:
        assert torch.all(dq[0, bq:min(2 * bq, nq), 0] == 0)


def test_backward_large_heads_xcd_runs():
    """Heads whose K and V take 138 MB (270,000 keys x 128 x bf16, twice) get the work order in
    runs of 32 items per XCD, in the forward and in both backward kernels: 4,220 query-block
    and 4,220 key-block items, so 16 whole runs of 256 and a partial last run in the natural
    order.  Rows keep 12 random key blocks of 2,110; the ragged last key block (48 keys) is
    kept by several rows and the ragged last query block keeps it.  dq on sampled rows (the
    last one included) and dk, dv on sampled key blocks (the last one included) against the
    oracle, to the small cases' bounds."""
    N, H, D, blk, per_row = 270_000, 2, 128, 128, 12
    scale = D ** -0.5
    nb = -(-N // blk)
    q, k, v, do = (rand((1, N, H, D), torch.bfloat16, s) for s in (90, 91, 92, 93))
    rng = np.random.default_rng(94)
    keep = np.zeros((nb, nb), bool)
    for r in range(nb):
        keep[r, rng.choice(nb, per_row, replace=False)] = True
    keep[rng.choice(nb - 1, 8, replace=False), nb - 1] = True
    keep[nb - 1, nb - 1] = True
    rp, ci = oracle.csr_from_bool(keep)
    rpd, cid = torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = vsa.vsa_block_sparse_attn_fwd(qd, kd, vd, rpd, cid, blk, blk, 1, scale)
    dq, dk, dv = vsa.vsa_block_sparse_attn_bwd(qd, kd, vd, o, dod, lse, rpd, cid, blk, blk, 1, scale)
    torch.cuda.synchronize()
    errs = {"dq": [], "dk": [], "dv": []}
    refs = {"dq": [], "dk": [], "dv": []}
    blocks = [(0, nb - 1), (1, int(rng.integers(nb - 1))), (1, int(rng.integers(nb - 1)))]
    for h in range(H):
        qh, kh, vh, dh = (t[0, :, h].double().numpy() for t in (q, k, v, do))
        rows = np.union1d(rng.choice(N, 96, replace=False), [N - 1])
        ref = oracle.attention_bwd_query_rows(qh[rows], rows, dh[rows], kh, vh, rp, ci, 0, blk, blk, scale)
        errs["dq"].append(np.abs(dq[0, rows, h].cpu().double().numpy() - ref))
        refs["dq"].append(np.abs(ref))
        for j in [j for hh, j in blocks if hh == h]:
            rk, rv = oracle.attention_bwd_key_block(j, qh, kh, vh, dh, rp, ci, 0, nb, blk, blk, scale)
            sl = slice(j * blk, min((j + 1) * blk, N))
            errs["dk"].append(np.abs(dk[0, sl, h].cpu().double().numpy() - rk))
            errs["dv"].append(np.abs(dv[0, sl, h].cpu().double().numpy() - rv))
            refs["dk"].append(np.abs(rk))
            refs["dv"].append(np.abs(rv))
    for name in ("dq", "dk", "dv"):
        e, r = np.concatenate(errs[name]), np.concatenate(refs[name])
        mx, mn = e.max() / r.max(), e.mean() / r.mean()
        print(f"large-head bwd {name}: max_norm {mx:.2e} mean_norm {mn:.2e}", flush=True)
        assert mx <= BWD_BF16_MAX and mn <= BWD_BF16_MEAN, name


@pytest.mark.parametrize("B,H,nq,nk,bq,bk,dens,per_head,dtype", [
    (2, 3, 700, 900, 128, 128, 0.5, True, torch.bfloat16),     # a mask per (batch, head), ragged blocks
    (2, 16, 1100, 2100, 64, 64, 0.4, True, torch.bfloat16),    # 544 key-block groups: grouped dK/dV
    (2, 2, 500, 600, 64, 64, 0.5, False, torch.float32),       # one shared mask, fp32 path
])
def test_attention_backward_two_batches(B, H, nq, nk, bq, bk, dens, per_head, dtype):
    """The backward with two batches against the oracle on every element."""
    D = 128
    scale = D ** -0.5
    q, k, v, do = (rand((B, n, H, D), dtype, 140 + i) for i, n in enumerate((nq, nk, nk, nq)))
    slabs = B * H if per_head else 1
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    rng = np.random.default_rng(145)
    keep = rng.random((slabs * nbq, nbk)) < dens
    keep[np.arange(slabs * nbq), rng.integers(0, nbk, size=slabs * nbq)] = True
    rp, ci = oracle.csr_from_bool(keep)
    rpd, cid = torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = vsa.vsa_block_sparse_attn_fwd(qd, kd, vd, rpd, cid, bq, bk, slabs, scale)
    dq, dk, dv = vsa.vsa_block_sparse_attn_bwd(qd, kd, vd, o, dod, lse, rpd, cid, bq, bk, slabs, scale)
    refs = oracle.attention_bwd(to_np(q), to_np(k), to_np(v), to_np(do), rp, ci, bq, bk, scale, slabs)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        err = np.abs(got.cpu().double().numpy() - ref)
        mx, mn = err.max() / np.abs(ref).max(), err.mean() / np.abs(ref).mean()
        print(f"two-batch bwd {B}x{H} {name}: max_norm {mx:.2e} mean_norm {mn:.2e}", flush=True)
        if dtype == torch.float32:
            assert mx <= BWD_F32_MAX, name
        else:
            assert mx <= BWD_BF16_MAX and mn <= BWD_BF16_MEAN, name
        for b in range(B):   # both batches carry gradient (nothing left at zero by an indexing slip)
            assert np.abs(got[b].cpu().double().numpy()).max() > 0, (name, b)


# ------------------------------------------------- grouped small query blocks
GROUPED_CASES = [
    # batch, heads, D, nq, nk, bq, bk, density, per-head masks
    (1, 48, 128, 2000, 2048, 64, 64, 0.5, True),     # 12 waves, 6 blocks per group; last group partial
    (1, 48, 64, 2000, 1900, 128, 128, 0.6, False),   # 12 waves, 3 blocks per group; shared mask
    (2, 20, 128, 1984, 2048, 128, 64, 0.4, True),    # 8 waves, 2 blocks per group; ragged last query block
    # 64-key blocks and smaller: two stream tiles per LDS stage
    (1, 48, 64, 1536, 1900, 64, 64, 0.5, True),      # 8 waves, 4 blocks per group; ragged last key block
    (2, 48, 64, 2000, 1000, 64, 32, 0.5, False),     # 12 waves, 32-key blocks (half-filled tiles)
    (1, 48, 64, 4000, 1000, 32, 64, 0.5, True),      # 32-row blocks: 12 per group
]


def test_union_lists_walk_fallback():
    """Groups whose row bitmaps do not fit the union kernel's LDS share (3 rows of 44,000
    one-key blocks) take the list walk instead; the grouped run still equals the ungrouped
    one bit for bit and matches the oracle."""
    B, H, D, nq, nk, bq, bk = 1, 32, 64, 3072, 44000, 128, 1
    scale = D ** -0.5
    q, k, v = rand((B, nq, H, D), torch.bfloat16, 80), rand((B, nk, H, D), torch.bfloat16, 81), \
        rand((B, nk, H, D), torch.bfloat16, 82)
    nbq, nbk = nq // bq, nk
    rng = np.random.default_rng(83)
    keep = rng.random((nbq, nbk)) < 0.005
    keep[np.arange(nbq), rng.integers(0, nbk, size=nbq)] = True
    rp, ci = oracle.csr_from_bool(keep)
    rpd, cid = torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    assert vsa.attn_fwd_workspace_bytes(qd, kd, rpd, cid, bq, bk, 1) > 0    # this case does group
    o_g, l_g = vsa.vsa_block_sparse_attn_fwd(qd, kd, vd, rpd, cid, bq, bk, 1, scale)
    o_u, l_u = vsa.vsa_block_sparse_attn_fwd(qd, kd, vd, rpd, cid, bq, bk, 1, scale, grouped=False)
    assert torch.equal(o_g, o_u) and torch.equal(l_g, l_u)
    rows = np.concatenate([np.arange(0, 2 * bq), rng.choice(nq, 64, replace=False), [nq - 1]])
    ref, _ = oracle.attention_rows(to_np(q[0, rows, 5]), rows, to_np(k[0, :, 5]), to_np(v[0, :, 5]),
                                   rp, ci, 0, bq, bk, scale)
    err = np.abs(o_g[0, rows, 5].cpu().double().numpy() - ref)
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN


@pytest.mark.parametrize("case", GROUPED_CASES, ids=[str(i) for i in range(len(GROUPED_CASES))])
def test_grouped_query_blocks(case):
    """Grouped runs (union of a group's kept blocks) equal ungrouped runs (bit for bit where
    both walk whole tiles), and sampled rows match the oracle."""
    B, H, D, nq, nk, bq, bk, dens, per_head = case
    slabs = B * H if per_head else 1
    scale = D ** -0.5
    q, k, v = rand((B, nq, H, D), torch.bfloat16, 70), rand((B, nk, H, D), torch.bfloat16, 71), \
        rand((B, nk, H, D), torch.bfloat16, 72)
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    rng = np.random.default_rng(73)
    keep = rng.random((slabs * nbq, nbk)) < dens
    keep[np.arange(slabs * nbq), rng.integers(0, nbk, size=slabs * nbq)] = True
    keep[1] = False                                           # an empty row
    rp, ci = oracle.csr_from_bool(keep)
    rpd, cid = torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    assert vsa.attn_fwd_workspace_bytes(qd, kd, rpd, cid, bq, bk, slabs) > 0   # this case does group
    o_g, l_g = vsa.vsa_block_sparse_attn_fwd(qd, kd, vd, rpd, cid, bq, bk, slabs, scale)
    o_u, l_u = vsa.vsa_block_sparse_attn_fwd(qd, kd, vd, rpd, cid, bq, bk, slabs, scale, grouped=False)
    # with its workspace the grouped run also packs V^T (nq >= nk, key blocks of a multiple of 64),
    # which the ungrouped run, without one, cannot: another summation order of the row sums
    same_v = not (nq >= nk and bk % 64 == 0)
    if bq > 64 and same_v:    # both walk each row's tiles whole and in the same order
        assert torch.equal(o_g, o_u) and torch.equal(l_g, l_u)
    else:          # (ungrouped 64-row blocks also split each tile between two waves)
        assert (o_g.float() - o_u.float()).abs().max() <= BF16_MAX
    errs = []
    for b, h in ((0, 0), (B - 1, H - 1), (0, H // 2)):
        rows = np.concatenate([np.arange(bq, 2 * bq), rng.choice(nq, 64, replace=False), [nq - 1]])
        base = 0 if slabs == 1 else (b * H + h) * nbq
        ref, _ = oracle.attention_rows(to_np(q[b, rows, h]), rows, to_np(k[b, :, h]), to_np(v[b, :, h]),
                                       rp, ci, base, bq, bk, scale)
        errs.append(np.abs(o_g[b, rows, h].cpu().double().numpy() - ref))
    err = np.concatenate(errs)
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN


# ------------------------------------------------ groups across frames (radial)
@pytest.mark.parametrize("T,S,block,B,H,per_head", [
    (12, 1000, 128, 1, 16, False),   # 7.8 blocks per frame: groups 7 blocks apart, a ragged last block
    (9, 768, 64, 1, 40, True),       # 12 blocks per frame, 64-row blocks (two tiles per stage), per-head masks
    (40, 300, 128, 1, 8, False),     # 2.3 blocks per frame: groups 2 apart
    (12, 640, 128, 2, 8, True),      # two batches, a mask per (batch, head)
])
def test_radial_grouping_across_frames(T, S, block, B, H, per_head):
    """vsa_radial_attn_fwd groups query blocks at the same place of consecutive frames; it
    computes the same thing as the plain forward (bit for bit for 65- to 128-row blocks,
    whose rows walk the same tiles in the same order), with the radial mask or any other."""
    n = T * S
    nb = -(-n // block)
    q, k, v = (rand((B, n, H, 128), torch.bfloat16, 95 + i) for i in range(3))
    if per_head:
        rng = np.random.default_rng(96)
        keep = rng.random((B * H * nb, nb)) < 0.4
        keep[np.arange(B * H * nb), rng.integers(0, nb, size=B * H * nb)] = True
        keep[1] = False
        rp_h, ci_h = oracle.csr_from_bool(keep)
        rp, ci = torch.from_numpy(rp_h).to(DEV), torch.from_numpy(ci_h).to(DEV)
        slabs = B * H
    else:
        rp, ci = vsa.vsa_mask_radial(T, S, block, DEV)
        rp_h, ci_h = csr_np(rp, ci)
        slabs = 1
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    assert vsa.attn_fwd_workspace_bytes_radial(qd, kd, rp, ci, block, S, slabs) > 0      # it groups
    o_f, l_f = vsa.vsa_radial_attn_fwd(qd, kd, vd, rp, ci, block, S, slabs)
    o_p, l_p = vsa.vsa_block_sparse_attn_fwd(qd, kd, vd, rp, ci, block, block, slabs)
    if block > 64:
        assert torch.equal(o_f, o_p) and torch.equal(l_f, l_p)
    else:
        assert (o_f.float() - o_p.float()).abs().max() <= BF16_MAX
    rng = np.random.default_rng(97)
    errs = []
    for b, h in ((0, 0), (B - 1, H - 1)):
        rows = np.concatenate([rng.choice(n, 96, replace=False), [n - 1]])
        base = 0 if slabs == 1 else (b * H + h) * nb
        ref, _ = oracle.attention_rows(to_np(q[b, rows, h]), rows, to_np(k[b, :, h]), to_np(v[b, :, h]),
                                       rp_h, ci_h, base, block, block, 128 ** -0.5)
        errs.append(np.abs(o_f[b, rows, h].cpu().double().numpy() - ref))
    err = np.concatenate(errs)
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN


# ------------------------------------------------------- split key streams
SPLIT_CASES = [
    # batch, heads, D, nq, nk, bq, bk, density, per-head masks
    (1, 4, 128, 2000, 3000, 64, 64, 0.5, True),      # 4-wave key split; ragged last query and key blocks
    (1, 2, 128, 1000, 5000, 128, 128, 0.6, False),   # 4 waves per 128-row block
    (2, 1, 64, 777, 9000, 384, 384, 0.7, True),      # 12-wave blocks; chunks of unequal length
    (1, 6, 128, 4680, 32760, 64, 64, 0.22, True),    # half the heads of the autoregressive chunk step
    (1, 2, 128, 2100, 2030, 64, 64, 0.6, True),      # nq >= nk: split with V packed transposed
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[str(i) for i in range(len(SPLIT_CASES))])
def test_split_key_streams(case):
    """Too few rows to fill the chip: each row's kept-block list is split over several
    workgroups and merged.  The result matches the oracle, equals the unsplit run to
    rounding, is the same on a second call, and an empty row still gives 0 and -inf."""
    B, H, D, nq, nk, bq, bk, dens, per_head = case
    slabs = B * H if per_head else 1
    scale = D ** -0.5
    q, k, v = rand((B, nq, H, D), torch.bfloat16, 90), rand((B, nk, H, D), torch.bfloat16, 91), \
        rand((B, nk, H, D), torch.bfloat16, 92)
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    rng = np.random.default_rng(93)
    keep = rng.random((slabs * nbq, nbk)) < dens
    keep[:, -1] |= rng.random(slabs * nbq) < 0.5                     # the ragged key block
    keep[np.arange(slabs * nbq), rng.integers(0, nbk, size=slabs * nbq)] = True
    keep[1] = False                                                    # an empty row
    keep[2, :3] = True                                                 # a short row: chunks may be empty
    keep[2, 3:] = False
    rp, ci = oracle.csr_from_bool(keep)
    rpd, cid = torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    label = __import__("bench").attn_kernel_name(D, bq, bk, True, B, H, nbq, False, nbk)
    assert label.split(", ")[6] == "true", label                      # this case does split
    o_s, l_s = vsa.vsa_block_sparse_attn_fwd(qd, kd, vd, rpd, cid, bq, bk, slabs, scale)
    o_s2, l_s2 = vsa.vsa_block_sparse_attn_fwd(qd, kd, vd, rpd, cid, bq, bk, slabs, scale)
    assert torch.equal(o_s, o_s2) and torch.equal(l_s, l_s2)
    o_u, l_u = vsa.vsa_block_sparse_attn_fwd(qd, kd, vd, rpd, cid, bq, bk, slabs, scale, grouped=False)
    assert (o_s.float() - o_u.float()).abs().max() <= BF16_MAX
    assert torch.allclose(l_s, l_u, rtol=0, atol=1e-4, equal_nan=False) or \
        torch.equal(torch.isinf(l_s), torch.isinf(l_u))
    errs = []
    for b, h in ((0, 0), (B - 1, H - 1)):
        rows = np.concatenate([np.arange(0, 3 * bq), rng.choice(nq, 64, replace=False), [nq - 1]])
        rows = rows[rows < nq]
        base = 0 if slabs == 1 else (b * H + h) * nbq
        ref, ref_lse = oracle.attention_rows(to_np(q[b, rows, h]), rows, to_np(k[b, :, h]), to_np(v[b, :, h]),
                                             rp, ci, base, bq, bk, scale)
        errs.append(np.abs(o_s[b, rows, h].cpu().double().numpy() - ref))
        got_lse = l_s[b, h, rows].cpu().double().numpy()
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(got_lse), fin)
        assert np.abs(got_lse[fin] - ref_lse[fin]).max() < 2e-2
    err = np.concatenate(errs)
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN
    if slabs > 1 or nbq > 1:                                           # the empty row: zeros
        assert torch.all(o_s[0, bq:min(2 * bq, nq), 0] == 0)


# ------------------------------------------------------------- tiled forward
# grid, tile, batch, heads, head_dim, dtype, mask (an STA window, or None: random per head)
TILED_CASES = [
    ((12, 16, 16), (6, 8, 8), 1, 2, 128, torch.bfloat16, (3, 3, 3)),   # 384-token tiles: 12-wave blocks
    ((12, 64, 64), (1, 8, 8), 1, 2, 64, torch.bfloat16, None),         # 64-token tiles: grouped / key split
    ((8, 8, 16), (4, 4, 4), 1, 3, 128, torch.bfloat16, None),          # th*tw = 16 divides 64
    ((4, 32, 16), (2, 16, 8), 1, 2, 128, torch.bfloat16, (1, 3, 3)),   # 256-token tiles: 8-wave blocks
    ((2, 4, 256), (1, 1, 128), 1, 2, 64, torch.bfloat16, (1, 1, 3)),   # tw a multiple of 64
    ((6, 8, 8), (3, 4, 4), 1, 2, 128, torch.bfloat16, None),           # 48-token tiles: one partial copy tile each
    ((12, 8, 16), (6, 4, 4), 2, 2, 64, torch.bfloat16, (3, 1, 3)),     # 96-token tiles: a full and a partial copy tile
    ((16, 16, 32), (16, 16, 16), 1, 2, 128, torch.bfloat16, None),     # 4,096-token tiles: all 64 copy-tile offsets
    ((4, 8, 8), (2, 4, 4), 2, 2, 64, torch.float32, None),             # fp32 path
]


@pytest.mark.parametrize("case", TILED_CASES, ids=[str(i) for i in range(len(TILED_CASES))])
def test_tiled_attention(case):
    """The forward on raster tokens with the tiles as blocks equals tile reorder ->
    forward -> inverse reorder bit for bit (o and lse, grouped and not), and sampled
    rows match the oracle."""
    grid, tile, B, H, D, dtype, window = case
    n, V = int(np.prod(grid)), int(np.prod(tile))
    n_tiles = n // V
    scale = D ** -0.5
    q, k, v = (rand((B, n, H, D), dtype, 80 + i) for i in range(3))
    if window is not None:
        rp, ci = oracle.mask_sta(grid, tile, window)
        slabs = 1
    else:
        slabs = B * H
        rng = np.random.default_rng(84)
        keep = rng.random((slabs * n_tiles, n_tiles)) < (0.4 if n_tiles < 100 else 0.1)
        keep[np.arange(slabs * n_tiles), rng.integers(0, n_tiles, size=slabs * n_tiles)] = True
        keep[2] = False                                           # an empty row
        rp, ci = oracle.csr_from_bool(keep)
    rpd, cid = torch.from_numpy(np.asarray(rp, np.int32)).to(DEV), torch.from_numpy(np.asarray(ci, np.int32)).to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    # raster position of tile-major position p
    perm = oracle.tile_reorder(np.arange(n).reshape(1, n, 1, 1), grid, tile)[0, :, 0, 0]
    qt, kt, vt = (vsa.vsa_tile_reorder(x, grid, tile) for x in (qd, kd, vd))
    if V == 64 and n_tiles >= 768:   # this case runs grouped
        assert vsa.tiled_attn_workspace_bytes(qd, grid, tile, rpd, cid, slabs) > 0
    for grouped in (True, False):
        o_t, l_t = vsa.vsa_tiled_attn_fwd(qd, kd, vd, grid, tile, rpd, cid, slabs, scale, grouped=grouped)
        o_r, l_r = vsa.vsa_block_sparse_attn_fwd(qt, kt, vt, rpd, cid, V, V, slabs, scale, grouped=grouped)
        assert torch.equal(o_t, vsa.vsa_tile_reorder(o_r, grid, tile, inverse=True))
        assert torch.equal(l_t[..., torch.from_numpy(perm).to(DEV)], l_r)
    qn, kn, vn = (oracle.tile_reorder(to_np(x), grid, tile) for x in (q, k, v))
    rng = np.random.default_rng(85)
    errs = []
    for b, h in ((0, 0), (B - 1, H - 1)):
        rows = np.concatenate([np.arange(min(V, 64)), rng.choice(n, 48, replace=False), [n - 1]])
        base = 0 if slabs == 1 else (b * H + h) * n_tiles
        ref, ref_lse = oracle.attention_rows(qn[b, rows, h], rows, kn[b, :, h], vn[b, :, h], rp, ci, base, V, V,
                                             scale)
        errs.append(np.abs(o_t[b, perm[rows], h].cpu().double().numpy() - ref))
        got_lse = l_t[b, h, perm[rows]].cpu().double().numpy()
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(got_lse), fin)
        assert np.abs(got_lse[fin] - ref_lse[fin]).max() < (1e-4 if dtype == torch.float32 else 2e-2)
    err = np.concatenate(errs)
    if dtype == torch.float32:
        assert err.max() <= F32_MAX
    else:
        assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN

"""GPU parity of each library call on small synthetic problems (all rows compared).

Every case goes through the C ABI (via the ctypes binding) and is compared with
the fp64 oracle on the same inputs: masks and reorders bit-exactly, attention to
the bf16 tolerance (max-abs 2e-2, mean-abs 2e-3) or 1e-4 for fp32."""
import numpy as np
import pytest
import torch

import block_sparse_attention_masks_amd as vsa
import oracle

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


def _compare_selected(rp, ci, orp, oci, exempt):
    bad = []
    for r in range(len(orp) - 1):
        a, b = ci[rp[r]:rp[r + 1]], oci[orp[r]:orp[r + 1]]
        if not np.array_equal(a, b) and not exempt[r]:
            bad.append(r)
    return bad


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
    orp, oci, flagged, ties = oracle.mask_nabla(to_np(q), to_np(k), bq, bk, scale, thr)
    assert len(rp) == len(orp)
    bad = _compare_selected(rp, ci, orp, oci, flagged | ties)
    assert not bad, f"rows differing outside the flagged set: {bad[:10]}"


@pytest.mark.parametrize("nk,bk,forced,topk", [
    (3000, 64, [(0, 5), (40, 47)], 6),
    (2000, 1, [(0, 25), (1900, 2000)], 16),     # 2,000 key blocks: 8 sort slots per thread
])
def test_mask_topk_forced_bit_exact(nk, bk, forced, topk):
    q = rand((2, 700, 2, 128), torch.bfloat16, 4)
    k = rand((2, nk, 2, 128), torch.bfloat16, 5)
    rp, ci = csr_np(*vsa.vsa_mask_nabla(q.to(DEV), k.to(DEV), 64, bk, 0.1, topk=topk, forced=forced))
    orp, oci, ties = oracle.mask_ar(to_np(q), to_np(k), 64, bk, 0.1, topk, forced)
    assert not _compare_selected(rp, ci, orp, oci, ties)
    assert set(np.diff(rp).tolist()) == {sum(hi - lo for lo, hi in forced) + topk}


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
    # attention over the compact cache is the same computation, tile for tile
    vc = vsa.vsa_kv_gather(v.to(DEV), slot, slabs, bk, n_out)
    o_full, l_full = vsa.vsa_block_sparse_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), rpd, cid, bq, bk, slabs)
    o_comp, l_comp = vsa.vsa_block_sparse_attn_fwd(q.to(DEV), kc, vc, rpd, cc, bq, bk, slabs)
    assert torch.equal(o_full, o_comp) and torch.equal(l_full, l_comp)


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


# ------------------------------------------------- grouped small query blocks
GROUPED_CASES = [
    # batch, heads, D, nq, nk, bq, bk, density, per-head masks
    (1, 48, 128, 2000, 2048, 64, 64, 0.5, True),     # 12 waves, 6 blocks per group; last group partial
    (1, 48, 64, 2000, 1900, 128, 128, 0.6, False),   # 12 waves, 3 blocks per group; shared mask
    (2, 20, 128, 2048, 2048, 128, 64, 0.4, True),    # 8 waves, 2 blocks per group
    # 64-key blocks and smaller: two stream tiles per LDS stage
    (1, 48, 64, 1536, 1900, 64, 64, 0.5, True),      # 8 waves, 4 blocks per group; ragged last key block
    (2, 48, 64, 2000, 1000, 64, 32, 0.5, False),     # 12 waves, 32-key blocks (half-filled tiles)
]


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
    if bq > 64:    # both walk each row's tiles whole and in the same order
        assert torch.equal(o_g, o_u) and torch.equal(l_g, l_u)
    else:          # ungrouped 64-row blocks split each tile between two waves: another summation order
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

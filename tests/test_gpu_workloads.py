"""GPU parity at the five workloads' full sizes, through the whole path.

Each test runs the path the benchmark times (tile reorder -> mask -> attention ->
inverse reorder; for the STA workloads the mask, then the attention with the reorder
folded in, checked bit for bit against the separate passes) on the seeded synthetic inputs, compares the mask with the fp64
oracle in full (bit-exact; NABLA / top-k rows whose decision sits within rounding
of the cut are flagged and counted; they are exempt only if the GPU's answer is still an
admissible cut, see tests/mask_parity.py), and compares the output with the
oracle fed the GPU's own mask: every row for the small workloads, 4,096 sampled
(head, query) rows for the three large ones."""
import time

import numpy as np
import pytest
import torch

import block_sparse_attention_masks_amd as vsa
import oracle
from mask_parity import check_nabla, check_topk
from workloads import gen
from workloads.configs import CONFIGS

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16_MAX, BF16_MEAN, F32_MAX = 2e-2, 2e-3, 1e-4


def log(*a):
    print(*a, flush=True)


def csr_np(rp, ci):
    rp = rp.cpu().numpy()
    return rp, ci[: int(rp[-1])].cpu().numpy()


def _sampled_rows_check(name, x_cpu, o_gpu, rp, ci, block_q, block_k, n_slabs, perm=None, n_rows=4096):
    """Oracle output of sampled (b, h, raster query token) rows vs the GPU output.

    perm (tile-major position -> raster token) describes the order the attention
    ran in; the oracle reorders its own copies of Q, K, V with it."""
    cfg = CONFIGS[name]
    D = cfg["head_dim"]
    scale = D ** -0.5
    rows = gen.sample_rows(name, n_rows)
    o_cpu = o_gpu.cpu()
    nbq = -(-x_cpu["q"].shape[1] // block_q)
    inv = None if perm is None else np.argsort(perm)
    errs = []
    for h in np.unique(rows[:, 1]):
        sel = rows[rows[:, 1] == h]
        b = 0
        qh = x_cpu["q"][b, :, h].double().numpy()
        kh = x_cpu["k"][b, :, h].double().numpy()
        vh = x_cpu["v"][b, :, h].double().numpy()
        if perm is not None:
            qh, kh, vh = qh[perm], kh[perm], vh[perm]
        toks = sel[:, 2]
        pos = toks if inv is None else inv[toks]          # row position in the attention order
        base = 0 if n_slabs == 1 else (b * cfg["heads"] + h) * nbq
        o_ref, _ = oracle.attention_rows(qh[pos], pos, kh, vh, rp, ci, base, block_q, block_k, scale)
        got = o_cpu[b, toks, h].double().numpy()
        errs.append(np.abs(got - o_ref))
    err = np.concatenate(errs)
    return err.max(), err.mean()


def _run_path(x, grid, tile, mask_fn, block, n_slabs, fused=False, frame_tokens=None):
    """reorder (if tiled) -> mask -> attention -> inverse reorder, on the GPU; fused: the
    mask, then the attention on raster-order tokens with the reorder folded in; with
    frame_tokens, the attention groups query blocks across frames (vsa_radial_attn_fwd)."""
    qd, kd, vd = (x[w].to(DEV) for w in ("q", "k", "v"))
    if fused:
        rp, ci = mask_fn(None, None)
        o, _ = vsa.vsa_tiled_attn_fwd(qd, kd, vd, grid, tile, rp, ci, n_slabs)
        torch.cuda.synchronize()
        return o, rp, ci
    if tile is not None:
        qd, kd, vd = (vsa.vsa_tile_reorder(t, grid, tile) for t in (qd, kd, vd))
    rp, ci = mask_fn(qd, kd)
    o, lse = vsa.vsa_block_sparse_attn_fwd(qd, kd, vd, rp, ci, block, block, n_slabs, frame_tokens=frame_tokens)
    if tile is not None:
        o = vsa.vsa_tile_reorder(o, grid, tile, inverse=True)
    torch.cuda.synchronize()
    return o, rp, ci


# ------------------------------------------------------------------------ tiny
@pytest.mark.parametrize("variant", ["dense", "sta", "nabla"])
def test_tiny_fp32(variant):
    cfg = CONFIGS["tiny"]
    grid, tile = cfg["grid"], cfg["tile"]
    x = gen.make_inputs("tiny")
    xq, xk, xv = (oracle.tile_reorder(x[w].double().numpy(), grid, tile) for w in ("q", "k", "v"))
    scale = 64 ** -0.5
    if variant == "dense":
        fn, slabs = (lambda q, k: vsa.all_ones_mask(32, 32, DEV)), 1
        orp, oci = oracle.mask_all(32, 32)
    elif variant == "sta":
        fn, slabs = (lambda q, k: vsa.vsa_mask_sta(grid, tile, cfg["sta_window"], DEV)), 1
        orp, oci = oracle.mask_sta(grid, tile, cfg["sta_window"])
    else:
        thr = cfg["nabla_threshold"]
        fn, slabs = (lambda q, k: vsa.vsa_mask_nabla(q, k, 64, 64, scale, threshold=thr)), 2
    o, rp_d, ci_d = _run_path(x, grid, tile, fn, 64, slabs)
    rp, ci = csr_np(rp_d, ci_d)
    if variant == "nabla":
        log(f"tiny/nabla mask: {check_nabla(rp, ci, xq, xk, 64, 64, scale, thr)}")
    else:
        assert np.array_equal(rp, orp) and np.array_equal(ci, oci)
    o_ref, _ = oracle.attention(xq, xk, xv, rp, ci, 64, 64, scale, slabs)
    o_ref = oracle.tile_reorder(o_ref, grid, tile, inverse=True)
    err = np.abs(o.cpu().double().numpy() - o_ref)
    log(f"tiny/{variant}: nnz={len(ci)} max_abs={err.max():.2e} mean_abs={err.mean():.2e}")
    assert err.max() <= F32_MAX


# ------------------------------------------------------------------------- sta
@pytest.mark.slow
@pytest.mark.timeout(600)
def test_sta_workload():
    cfg = CONFIGS["sta"]
    grid, tile, window = cfg["grid"], cfg["tile"], cfg["window"]
    t0 = time.time()
    x = gen.make_inputs("sta")
    log(f"sta: inputs {time.time() - t0:.1f}s")
    mask = lambda q, k: vsa.vsa_mask_sta(grid, tile, window, DEV)
    o, rp_d, ci_d = _run_path(x, grid, tile, mask, 384, 1, fused=True)
    o_sep, _, _ = _run_path(x, grid, tile, mask, 384, 1)
    assert torch.equal(o, o_sep)   # the folded reorder moves the same rows
    del o_sep
    rp, ci = csr_np(rp_d, ci_d)
    orp, oci = oracle.mask_sta(grid, tile, window)
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci) and len(ci) == 9152
    perm = oracle.tile_order_source(grid, tile)
    mx, mn = _sampled_rows_check("sta", x, o, rp, ci, 384, 384, 1, perm=perm)
    log(f"sta: 4096 rows max_abs={mx:.2e} mean_abs={mn:.2e} ({time.time() - t0:.1f}s)")
    assert mx <= BF16_MAX and mn <= BF16_MEAN


# ----------------------------------------------------------------------- nabla
@pytest.mark.slow
@pytest.mark.timeout(900)
def test_nabla_workload():
    cfg = CONFIGS["nabla"]
    grid, tile, thr = cfg["grid"], cfg["tile"], cfg["threshold"]
    scale = 128 ** -0.5
    t0 = time.time()
    x = gen.make_inputs("nabla")
    log(f"nabla: inputs {time.time() - t0:.1f}s")
    fn = lambda q, k: vsa.vsa_mask_nabla(q, k, 64, 64, scale, threshold=thr)
    o, rp_d, ci_d = _run_path(x, grid, tile, fn, 64, 40)
    rp, ci = csr_np(rp_d, ci_d)
    perm = oracle.tile_order_source(grid, tile)
    qt = x["q"][:, perm].double().numpy()
    kt = x["k"][:, perm].double().numpy()
    counts = check_nabla(rp, ci, qt, kt, 64, 64, scale, thr)
    del qt, kt
    dens = np.diff(rp).reshape(40, 960).sum(axis=1) / (960 * 960)
    log(f"nabla mask: {counts}; density per head min {dens.min():.3f} max {dens.max():.3f} "
        f"(sparsity {1 - dens.mean():.3f})")
    mx, mn = _sampled_rows_check("nabla", x, o, rp, ci, 64, 64, 40, perm=perm)
    log(f"nabla: 4096 rows max_abs={mx:.2e} mean_abs={mn:.2e} ({time.time() - t0:.1f}s)")
    assert mx <= BF16_MAX and mn <= BF16_MEAN


# ---------------------------------------------------------------------- radial
@pytest.mark.slow
@pytest.mark.timeout(900)
def test_radial_workload():
    cfg = CONFIGS["radial"]
    T, H, W = cfg["grid"]
    S, block = H * W, cfg["block"]
    t0 = time.time()
    x = gen.make_inputs("radial")
    log(f"radial: inputs {time.time() - t0:.1f}s")
    o, rp_d, ci_d = _run_path(x, None, None, lambda q, k: vsa.vsa_mask_radial(T, S, block, DEV), block, 1,
                              frame_tokens=S)
    rp, ci = csr_np(rp_d, ci_d)
    orp, oci = oracle.mask_radial(T, S, block)
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci) and len(ci) == 2718652
    mx, mn = _sampled_rows_check("radial", x, o, rp, ci, block, block, 1)
    log(f"radial: 4096 rows max_abs={mx:.2e} mean_abs={mn:.2e} ({time.time() - t0:.1f}s)")
    assert mx <= BF16_MAX and mn <= BF16_MEAN


# ---------------------------------------------------------------------- ar
@pytest.mark.slow
@pytest.mark.timeout(600)
def test_ar_chunk_workload():
    cfg = CONFIGS["ar"]
    T, H, W = cfg["grid"]
    block, topk = cfg["block"], cfg["topk"]
    scale = 128 ** -0.5
    forced = vsa.ar_forced_ranges(H * W, T, cfg["anchor_frames"], cfg["recent_frames"], block)
    assert forced == oracle.ar_forced_ranges(H * W, T, cfg["anchor_frames"], cfg["recent_frames"], block)
    x = gen.make_inputs("ar")
    fn = lambda q, k: vsa.vsa_mask_nabla(q, k, block, block, scale, topk=topk, forced=forced)
    o, rp_d, ci_d = _run_path(x, None, None, fn, block, 12)
    rp, ci = csr_np(rp_d, ci_d)
    xq, xk, xv = (x[w].double().numpy() for w in ("q", "k", "v"))
    counts, _ = check_topk(rp, ci, xq, xk, block, block, scale, topk, forced)
    log(f"ar mask: {counts}")
    assert set(np.diff(rp).tolist()) == {115}
    o_ref, _ = oracle.attention(xq, xk, xv, rp, ci, block, block, scale, 12)
    err = np.abs(o.cpu().double().numpy() - o_ref)
    log(f"ar: all rows max_abs={err.max():.2e} mean_abs={err.mean():.2e}")
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN


# ------------------------------------------------------------- composition
@pytest.mark.slow
@pytest.mark.timeout(600)
def test_sta_heads_workload():
    cfg = CONFIGS["sta_heads"]
    grid, tile, H = cfg["grid"], cfg["tile"], cfg["heads"]
    wins = [cfg["windows"][h % len(cfg["windows"])] for h in range(H)]
    t0 = time.time()
    x = gen.make_inputs("sta_heads")
    mask = lambda q, k: vsa.vsa_mask_sta_heads(grid, tile, wins, DEV)
    o, rp_d, ci_d = _run_path(x, grid, tile, mask, 384, H, fused=True)
    o_sep, _, _ = _run_path(x, grid, tile, mask, 384, H)
    assert torch.equal(o, o_sep)   # the folded reorder moves the same rows
    del o_sep
    rp, ci = csr_np(rp_d, ci_d)
    orp, oci = oracle.mask_sta_heads(grid, tile, wins, 1)
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci)
    perm = oracle.tile_order_source(grid, tile)
    mx, mn = _sampled_rows_check("sta_heads", x, o, rp, ci, 384, 384, H, perm=perm)
    log(f"sta_heads: nnz={len(ci)} 4096 rows max_abs={mx:.2e} mean_abs={mn:.2e} ({time.time() - t0:.1f}s)")
    assert mx <= BF16_MAX and mn <= BF16_MEAN


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_nabla_sta_workload():
    cfg = CONFIGS["nabla_sta"]
    grid, tile, thr, window = cfg["grid"], cfg["tile"], cfg["threshold"], cfg["window"]
    H = cfg["heads"]
    scale = 128 ** -0.5
    t0 = time.time()
    x = gen.make_inputs("nabla_sta")

    parts = {}

    def fn(q, k):
        parts["nabla"] = vsa.vsa_mask_nabla(q, k, 64, 64, scale, threshold=thr)
        rps, cis = vsa.vsa_mask_sta(grid, tile, window, DEV)
        return vsa.vsa_mask_union(*parts["nabla"], H, rps, cis, 1, 960, 960)
    o, rp_d, ci_d = _run_path(x, grid, tile, fn, 64, H)
    rp, ci = csr_np(rp_d, ci_d)
    rpn, cin = csr_np(*parts["nabla"])
    perm = oracle.tile_order_source(grid, tile)
    qt = x["q"][:, perm].double().numpy()
    kt = x["k"][:, perm].double().numpy()
    counts = check_nabla(rpn, cin, qt, kt, 64, 64, scale, thr)      # the NABLA part, as for nabla
    del qt, kt
    # the union, bit for bit, of the GPU's NABLA mask and the oracle's STA window
    orp_s, oci_s = oracle.mask_sta(grid, tile, window)
    orp, oci = oracle.mask_union(rpn, cin, H, orp_s, oci_s, 1, 960)
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci)
    log(f"nabla_sta: nnz={len(ci)} (nabla alone {len(cin)}); nabla mask {counts}")
    mx, mn = _sampled_rows_check("nabla_sta", x, o, rp, ci, 64, 64, H, perm=perm)
    log(f"nabla_sta: 4096 rows max_abs={mx:.2e} mean_abs={mn:.2e} ({time.time() - t0:.1f}s)")
    assert mx <= BF16_MAX and mn <= BF16_MEAN


# ------------------------------------------------------------------------ SICS
@pytest.mark.slow
@pytest.mark.timeout(600)
def test_sics_sta_workload():
    """SICS scores of the tile-reordered K of the sta workload (24 heads x 300 blocks of
    384 tokens); the oracle's pairwise definition on 240 sampled (head, block) pairs."""
    cfg = CONFIGS["sta"]
    grid, tile = cfg["grid"], cfg["tile"]
    x = gen.make_inputs("sta")
    kd = vsa.vsa_tile_reorder(x["k"].to(DEV), grid, tile)
    got = vsa.vsa_block_sics(kd, 384).cpu().numpy()
    perm = oracle.tile_order_source(grid, tile)
    kt = x["k"][:, perm]
    rng = np.random.default_rng(41)
    worst = 0.0
    for h, i in zip(rng.integers(0, 24, 240), rng.integers(0, 300, 240)):
        rows = kt[:, i * 384:(i + 1) * 384, h:h + 1].double().numpy()
        want = oracle.block_sics(rows, 384)[0, 0, 0]
        worst = max(worst, abs(got[0, h, i] - want) / want)
    log(f"sics/sta: score range {got.min():.1f}..{got.max():.1f}, worst relative error {worst:.2e}")
    assert worst < 1e-10


# ------------------------------------------------------------- KV compaction
@pytest.mark.timeout(600)
def test_ar_kv_compaction_workload():
    """The ar chunk's KV cache compacted to the blocks its heads keep: the slot map equals
    the oracle's on the GPU's mask, and attention over the compact cache equals
    attention over the full cache bit for bit."""
    from oracle import kvcache
    cfg = CONFIGS["ar"]
    T, Hg, Wg = cfg["grid"]
    block, topk, H = cfg["block"], cfg["topk"], cfg["heads"]
    scale = 128 ** -0.5
    forced = vsa.ar_forced_ranges(Hg * Wg, T, cfg["anchor_frames"], cfg["recent_frames"], block)
    x = gen.make_inputs("ar")
    q, k, v = (x[w].to(DEV) for w in ("q", "k", "v"))
    rp, ci = vsa.vsa_mask_nabla(q, k, block, block, scale, topk=topk, forced=forced)
    nq, nk = q.shape[1], k.shape[1]
    nbq, nbk = -(-nq // block), -(-nk // block)
    kc, vc, cc, n_out, slot, info = vsa.vsa_kv_compact(k, v, rp, ci, H, block, block)
    rph, cih = csr_np(rp, ci)
    _, remap, n_full_max, has_tail = kvcache.kv_keep(rph, cih, H, nbq, nbk, nk, block)
    assert np.array_equal(slot.cpu().numpy(), remap)
    assert n_out == kvcache.compact_tokens(n_full_max, has_tail, nk, block)
    kept = (remap >= 0).sum(axis=1)
    log(f"ar kv: cache {nk} -> {n_out} tokens ({100 * (1 - n_out / nk):.1f}% smaller), kept blocks per head "
        f"{kept.min()}..{kept.max()} of {nbk}")
    o_full, l_full = vsa.vsa_block_sparse_attn_fwd(q, k, v, rp, ci, block, block, H, scale)
    o_comp, l_comp = vsa.vsa_block_sparse_attn_fwd(q, kc, vc, rp, cc, block, block, H, scale)
    assert torch.equal(o_full, o_comp) and torch.equal(l_full, l_comp)


# ------------------------------------------------------------------ backward
@pytest.mark.slow
@pytest.mark.timeout(900)
def test_backward_sta_workload():
    """Gradients at the sta workload's full size (tile order, as the path runs): dq on 512
    sampled (head, query) rows and dk, dv on 3 sampled (head, key block) pairs, each
    from the oracle's own sampled evaluation."""
    cfg = CONFIGS["sta"]
    grid, tile, window = cfg["grid"], cfg["tile"], cfg["window"]
    H, D, blk = cfg["heads"], cfg["head_dim"], 384
    scale = D ** -0.5
    t0 = time.time()
    x = gen.make_inputs("sta")
    perm = oracle.tile_order_source(grid, tile)
    qt, kt, vt = (x[w][:, perm].contiguous() for w in ("q", "k", "v"))
    dout = (torch.randn(qt.shape, generator=torch.Generator().manual_seed(77), dtype=torch.float32)
            .to(torch.bfloat16))
    qd, kd, vd, dd = (t.to(DEV) for t in (qt, kt, vt, dout))
    rp_d, ci_d = vsa.vsa_mask_sta(grid, tile, window, DEV)
    o, lse = vsa.vsa_block_sparse_attn_fwd(qd, kd, vd, rp_d, ci_d, blk, blk, 1, scale)
    dq, dk, dv = vsa.vsa_block_sparse_attn_bwd(qd, kd, vd, o, dd, lse, rp_d, ci_d, blk, blk, 1, scale)
    torch.cuda.synchronize()
    rp, ci = csr_np(rp_d, ci_d)
    log(f"sta bwd: GPU done {time.time() - t0:.1f}s")
    rng = np.random.default_rng(78)
    nq = qt.shape[1]
    heads = rng.choice(H, 4, replace=False)
    errs = {"dq": [], "dk": [], "dv": []}
    refs = {"dq": [], "dk": [], "dv": []}
    for h in heads:
        qh, kh, vh, dh = (t[0, :, h].double().numpy() for t in (qt, kt, vt, dout))
        rows = np.sort(rng.choice(nq, 128, replace=False))
        ref = oracle.attention_bwd_query_rows(qh[rows], rows, dh[rows], kh, vh, rp, ci, 0, blk, blk, scale)
        errs["dq"].append(np.abs(dq[0, rows, h].cpu().double().numpy() - ref))
        refs["dq"].append(np.abs(ref))
    for h, j in zip(heads[:3], rng.choice(300, 3, replace=False)):
        qh, kh, vh, dh = (t[0, :, h].double().numpy() for t in (qt, kt, vt, dout))
        rk, rv = oracle.attention_bwd_key_block(j, qh, kh, vh, dh, rp, ci, 0, 300, blk, blk, scale)
        sl = slice(j * blk, (j + 1) * blk)
        errs["dk"].append(np.abs(dk[0, sl, h].cpu().double().numpy() - rk))
        errs["dv"].append(np.abs(dv[0, sl, h].cpu().double().numpy() - rv))
        refs["dk"].append(np.abs(rk))
        refs["dv"].append(np.abs(rv))
    for name in ("dq", "dk", "dv"):
        e, r = np.concatenate(errs[name]), np.concatenate(refs[name])
        mx, mn = e.max() / r.max(), e.mean() / r.mean()
        log(f"sta bwd {name}: max_norm {mx:.2e} mean_norm {mn:.2e}")
        # As for the small cases (P, dS rounded to bf16: 2^-9 per term), except that here D
        # = sum dO * O is built from the forward's bf16 O and enters dS un-cancelled while dq
        # is a difference of near-equal terms: the positional code (|P|^2 = 144) makes the keys
        # large and attention peaked, which amplifies that rounding relative to |dq| (x2.5
        # measured), so the mean bound is 4 * 2^-9.
        assert mx <= 8 * 2.0 ** -9 and mn <= 4 * 2.0 ** -9, name
    log(f"sta bwd: done {time.time() - t0:.1f}s")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_backward_radial_workload():
    """dq at the radial workload's full size, as the bench times it (the shared radial mask,
    the frame-grouped forward, then the backward in its XCD-run work order): 4 heads x 64
    sampled query rows, the ragged last token among them, each against the oracle's own
    evaluation of that row.  dk and dv are not sampled here: an oracle key block of this mask
    needs the full softmax of the ~100,000 query rows that keep it (a teraflop in fp64); the
    270,000-key test in test_gpu_kernels covers those kernels in the same work order."""
    cfg = CONFIGS["radial"]
    T, Hg, Wg = cfg["grid"]
    S, blk, H, D = Hg * Wg, cfg["block"], cfg["heads"], cfg["head_dim"]
    scale = D ** -0.5
    t0 = time.time()
    x = gen.make_inputs("radial")
    qd, kd, vd = (x[w].to(DEV) for w in ("q", "k", "v"))
    gd = torch.Generator(device=DEV).manual_seed(79)
    dd = torch.randn(qd.shape, generator=gd, device=DEV).to(torch.bfloat16)
    rp_d, ci_d = vsa.vsa_mask_radial(T, S, blk, DEV)
    o, lse = vsa.vsa_radial_attn_fwd(qd, kd, vd, rp_d, ci_d, blk, S)
    dq, dk, dv = vsa.vsa_block_sparse_attn_bwd(qd, kd, vd, o, dd, lse, rp_d, ci_d, blk, blk, 1, scale)
    torch.cuda.synchronize()
    del dk, dv
    rp, ci = csr_np(rp_d, ci_d)
    orp, oci = oracle.mask_radial(T, S, blk)
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci)
    log(f"radial bwd: GPU done {time.time() - t0:.1f}s")
    rng = np.random.default_rng(80)
    nq = qd.shape[1]
    errs, refs = [], []
    for h in rng.choice(H, 4, replace=False):
        rows = np.sort(rng.choice(nq - 1, 63, replace=False))
        rows = np.append(rows, nq - 1)                        # the ragged last block's last row
        qh, kh, vh = (x[w][0, :, h].double().numpy() for w in ("q", "k", "v"))
        dh = dd[0, rows, h].cpu().double().numpy()
        ref = oracle.attention_bwd_query_rows(qh[rows], rows, dh, kh, vh, orp, oci, 0, blk, blk, scale)
        errs.append(np.abs(dq[0, rows, h].cpu().double().numpy() - ref))
        refs.append(np.abs(ref))
    e, r = np.concatenate(errs), np.concatenate(refs)
    mx, mn = e.max() / r.max(), e.mean() / r.mean()
    log(f"radial bwd dq: max_norm {mx:.2e} mean_norm {mn:.2e} ({time.time() - t0:.1f}s)")
    # the bounds of the sta workload's backward, for the same reason: D built from the
    # forward's bf16 O enters dS while dq is a difference of near-equal terms under the
    # positional code's peaked attention
    assert mx <= 8 * 2.0 ** -9 and mn <= 4 * 2.0 ** -9

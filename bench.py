"""Benchmark of the block-sparse 3D-video attention path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input, all on
the GPU with the inputs resident in HBM:
    [tile reorder of Q, K, V] -> block mask -> block-sparse attention ->
    [inverse reorder of O]
For the STA workloads (sta, sta_heads) the reorder is folded into the attention
kernel's row addresses (vsa_tiled_attn_fwd on raster-order tokens): the step is
the mask, then that call; --unfused runs the separate passes instead.
The default workload is the radial one, the largest (24 heads, head_dim 128, bf16,
125x45x80 = 450,000 tokens, 3,600 per frame, raster 128-token blocks, radial
energy-decay mask; the attention runs as vsa_radial_attn_fwd, query blocks at the
same place of consecutive frames grouped); --workload sta | nabla | ar | nabla_sta | sta_heads |
ar_compact measures the others (their lines are reports, not the headline).

value       = kept-block attention FLOPs (4 * D * sum of nq*nk over kept block
              pairs, true token counts) / wall time of a step, TFLOP/s.
roofline    = the attention kernel alone: the same FLOPs / its mean launch time
              measured with HIP events on its stream, against the bf16 dense
              MFMA peak (2.5 PFLOP/s).
speedup     = the same kernel on an all-ones mask (dense attention) / sparse.
cpu_baseline= the fp64 oracle on the same path: its mask in full, its attention on
              sampled query blocks, extrapolated linearly in kept pairs to the
              whole path (FLOPs counted the same way); it also compares the
              oracle's mask with the GPU's, row by row.
hbm_passes  = SICS scores, the NABLA block mean-pool and (tiled workloads) the tile
              reorder, each timed alone with the caches flushed before every rep.
sclk        = the GFX clock (amdsmi, mean over the XCDs) while the attention kernel
              runs back to back for --clock-s seconds after the timed steps; the
              roofline's frac_at_measured_sclk scales the peak by it / 2.4 GHz.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload radial]
                       [--no-dense] [--no-cpu] [--no-bwd] [--unfused] [--clock-s S]
"""
import argparse
import hashlib
import json
import os
import sys
import threading
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
METRIC = "block-sparse attn effective TFLOPS (kept blocks), % bf16 MFMA peak; speedup vs dense"
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_masks_amd", "csrc", "attn_fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_{}_traffic.json")

DESCRIPTION = {
    "sta": "sta: 1 x 24 heads x 115,200 tokens (30x48x80 grid), head_dim 128, bf16, 6x8x8 tiles "
           "(384-token blocks), 3x3x5 tile window clipped at the border",
    "nabla": "nabla: 1 x 40 heads x 61,440 tokens (16x48x80 grid), head_dim 128, bf16, 1x8x8 tiles "
             "(64-token blocks), pooled-map CDF threshold 0.8, per-head masks",
    "radial": "radial: 1 x 24 heads x 450,000 tokens (125x45x80 grid, 3,600 per frame), head_dim 128, "
              "bf16, raster 128-token blocks, radial energy-decay mask",
    "nabla_sta": "nabla_sta: the nabla workload with its per-head NABLA masks united with a 3x3x5 STA "
                 "window on the 16x6x10 tile grid",
    "sta_heads": "sta_heads: the sta workload with one tile window per head (3x3x5, 1x3x3, 3x5x7 cycling "
                 "over the 24 heads)",
    "ar_compact": "ar_compact: the ar workload with its KV cache compacted to the blocks each head keeps "
                  "(plan, gather K and V, mask remap) before attention",
    "ar": "ar: 1 x 12 heads, 4,680 query tokens (3x30x52 chunk) over a 32,760-token KV cache "
          "(21x30x52), head_dim 128, bf16, 64-token blocks, anchors + last 3 frames + top-16",
}


def attn_flops(rp, ci, block_q, block_k, nq, nk, D, bh, n_slabs):
    """4*D*sum over kept (i, j) of nq(i)*nk(j) with true (ragged) token counts, over
    all bh = batch*heads (a shared mask, n_slabs = 1, counts once per (b, h))."""
    rp = np.asarray(rp, dtype=np.int64)
    ci = np.asarray(ci, dtype=np.int64)
    nbq = -(-nq // block_q)
    qsz = np.minimum(block_q, nq - np.arange(nbq) * block_q)
    ksz = np.minimum(block_k, nk - ci * block_k)
    csum = np.concatenate([[0], np.cumsum(ksz)])
    per_row = csum[rp[1:]] - csum[rp[:-1]]            # kept key tokens per CSR row
    total = float((per_row * np.tile(qsz, n_slabs)).sum())
    return 4.0 * D * total * (bh if n_slabs == 1 else 1)


def attn_kernel_name(D, block_q, block_k, grouped=False, batch=1, heads=1, n_qblocks=1, tiled=False,
                     n_kblocks=0, nq=0, nk=1):
    """Label of the bf16 instantiation the library launches (its plan, mirrored here).  With a
    workspace (grouped=True), query blocks of <= 128 rows are grouped into 12-, 8- or 4-wave
    workgroups, the first width whose group count keeps enough workgroups; otherwise it picks
    a 4-wave key split (<= 64 rows) or 12-, 8- or 4-wave workgroups from block_q, and, with a
    workspace, splits each row's key stream into chunks when the rows cannot fill one round
    of workgroups.  Template arguments: head_dim, key split, waves, grouped, tiled
    (raster-order tokens with the tiles as blocks), stream tiles per LDS stage (two for
    grouped, untiled key blocks of <= 64), split key streams, V packed transposed (with a
    workspace, key blocks of a multiple of 64 and nq >= nk)."""
    tl = str(tiled).lower()
    vt = str(bool(grouped and block_k % 64 == 0 and nq >= nk)).lower()
    if grouped:
        wpb = -(-block_q // 32)
        for nw in (12, 8, 4):
            G = nw // wpb
            if nw % wpb or G < 2:
                continue
            if batch * heads * -(-n_qblocks // G) >= (512 if nw == 4 else 256):
                tw = 2 if nw >= 8 and block_k <= 64 and not tiled else 1
                return f"attn_fwd_bf16_kernel<{D}, 1, {nw}, true, {tl}, {tw}, false, {vt}>"
    ks = 2 if block_q <= 64 else 1
    nw = 4 if ks == 2 else (12 if block_q % 384 == 0 else (8 if block_q % 256 == 0 else 4))
    items = batch * heads * n_qblocks * -(-block_q // (32 * nw // ks))
    slots = 256 * (2 if nw == 4 else 1)
    n = min(-(-2 * slots // items), 8, n_kblocks // 8)
    sp = grouped and items < slots and n_kblocks >= 16 and n >= 2
    return f"attn_fwd_bf16_kernel<{D}, {ks}, {nw}, false, {tl}, 1, {str(sp).lower()}, {vt}>"


def source_hash(path):
    """Hash of a kernel source's code: comments and blank space are dropped, so the stored
    traffic figure stays keyed to the code the counters measured."""
    import re
    with open(path) as f:
        text = f.read()
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"\s+", " ", text).strip()
    return hashlib.sha256(text.encode()).hexdigest()[:16]


class ClockSampler:
    """Samples the graphics clock of the first GPU (amdsmi, current GFX clock in MHz) from a
    background thread.  The published peaks assume 2.4 GHz; under a long matrix-core load the
    clock runs lower, and the sampled clock says how much.  The firmware's reading lags the
    load by some tens of milliseconds, so `result()` keeps the second half of the samples of
    a window in which the load runs without a break.  Any failure (no amdsmi, no permission)
    leaves the result's mean as None with the reason."""

    SPEC_MHZ = 2400.0

    def __init__(self, interval_s=0.01):
        self.interval_s, self.samples, self.error = interval_s, [], None
        self._stop, self._thread, self._amdsmi, self._handle = threading.Event(), None, None, None

    def __enter__(self):
        # amdsmi is opened, read and closed on the sampling thread, so that a stuck driver
        # query can only lose the reading, never hold up the benchmark
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()
        return self

    def _read(self):
        # the mean over the XCDs' current clocks (they differ by a few percent), else the
        # first XCD's from the clock query
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
        clks = [float(c) for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 65535]
        if clks:
            return sum(clks) / len(clks)
        info = self._amdsmi.amdsmi_get_clock_info(self._handle, self._amdsmi.AmdSmiClkType.GFX)
        return float(info["clk"])

    def _run(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
        except Exception as e:  # noqa: BLE001 -- reported, never fatal
            self.error = f"{type(e).__name__}: {e}"[:200]
            return
        self._amdsmi = amdsmi
        try:
            self._handle = amdsmi.amdsmi_get_processor_handles()[0]
            while not self._stop.is_set():
                self.samples.append(self._read())
                self._stop.wait(self.interval_s)
        except Exception as e:  # noqa: BLE001
            self.error = f"{type(e).__name__}: {e}"[:200]
        finally:
            try:
                amdsmi.amdsmi_shut_down()
            except Exception:  # noqa: BLE001
                pass

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=5.0)
            if self._thread.is_alive():
                self.error = "amdsmi did not answer within 5 s"
        return False

    def result(self, what):
        kept = self.samples[len(self.samples) // 2:]
        if not kept:
            return {"mean_mhz": None, "error": self.error or "no samples"}
        return {"mean_mhz": round(float(np.mean(kept)), 1), "min_mhz": round(min(kept), 1),
                "max_mhz": round(max(kept), 1), "samples": len(kept),
                "source": f"amdsmi: current GFX clock averaged over the XCDs of GPU 0, sampled every "
                          f"{self.interval_s * 1e3:.0f} ms while {what}; second half of the samples"}


def _oracle_mask(name, cfg, qt, kt):
    """The oracle's mask of a workload: (row_ptr, col_idx, flagged rows or None).  qt, kt:
    fp64 [B, N, heads, D] in the attention order (only the NABLA and top-k masks read them)."""
    import oracle
    D = cfg["head_dim"]
    if name == "sta":
        return (*oracle.mask_sta(cfg["grid"], cfg["tile"], cfg["window"]), None)
    if name == "sta_heads":
        wins = [cfg["windows"][h % len(cfg["windows"])] for h in range(cfg["heads"])]
        return (*oracle.mask_sta_heads(cfg["grid"], cfg["tile"], wins, cfg["batch"]), None)
    if name == "radial":
        T, Hg, Wg = cfg["grid"]
        return (*oracle.mask_radial(T, Hg * Wg, cfg["block"]), None)
    if name in ("nabla", "nabla_sta"):
        bq = cfg["tile"][0] * cfg["tile"][1] * cfg["tile"][2]
        rp, ci, fl, _ = oracle.mask_nabla(qt, kt, bq, bq, D ** -0.5, cfg["threshold"])
        if name == "nabla_sta":
            nbq = len(rp) // (cfg["batch"] * cfg["heads"])
            rps, cis = oracle.mask_sta(cfg["grid"], cfg["tile"], cfg["window"])
            rp, ci = oracle.mask_union(rp, ci, cfg["batch"] * cfg["heads"], rps, cis, 1, nbq)
        return rp, ci, fl
    T, Hg, Wg = cfg["grid"]
    forced = oracle.ar_forced_ranges(Hg * Wg, T, cfg["anchor_frames"], cfg["recent_frames"], cfg["block"])
    rp, ci, ties = oracle.mask_ar(qt, kt, cfg["block"], cfg["block"], D ** -0.5, cfg["topk"], forced)
    return rp, ci, ties


def _mask_rows_differ(rp_a, ci_a, rp_b, ci_b):
    """bool per row: the two CSR masks keep different blocks."""
    la, lb = np.diff(rp_a), np.diff(rp_b)
    out = la != lb
    for r in np.nonzero(~out)[0]:
        out[r] = not np.array_equal(ci_a[rp_a[r]:rp_a[r + 1]], ci_b[rp_b[r]:rp_b[r + 1]])
    return out


def cpu_baseline(name, cfg, x, path, rp_gpu, ci_gpu, flops_total, target_s=15.0):
    """The fp64 oracle on the same path, on a bounded sample.

    The mask is computed in full (the tile reorder of Q and K it needs included); the
    attention runs on runs of 16 consecutive query blocks, head by head in a seeded order,
    each head's Q, K, V converted to fp64 and tile-reordered, and the output rows reordered
    back, until about target_s seconds have run (every block at the small autoregressive
    shape).  The full path's time is extrapolated: t_mask + t_setup * heads / heads seen +
    t_runs * (all kept pairs / sampled pairs), and the rate is the path's kept-block FLOPs
    over that time.
    As a by-product the oracle's mask is compared row by row with the GPU's."""
    import oracle
    from threadpoolctl import threadpool_info
    B, H, D = cfg["batch"], cfg["heads"], cfg["head_dim"]
    scale = D ** -0.5
    bq, bk = path.bq, path.bk
    nq, nk = path.nq, path.nk
    perm = oracle.tile_order_source(cfg["grid"], cfg["tile"]) if path.tiled else None
    dyn = name in ("nabla", "nabla_sta", "ar", "ar_compact")
    # mask stage (timed): reorder of Q and K for the dynamic masks, then the mask
    t0 = time.perf_counter()
    qt = kt = None
    if dyn:
        qt, kt = (x[w].double().numpy() for w in ("q", "k"))
        if perm is not None:
            qt, kt = qt[:, perm], kt[:, perm]
    rp, ci, flags = _oracle_mask(name, cfg, qt, kt)
    t_mask = time.perf_counter() - t0
    del qt, kt
    check = {"rows": int(len(rp) - 1), "rows_differ": None}
    if len(rp) == len(rp_gpu):
        diff = _mask_rows_differ(rp, ci, rp_gpu, ci_gpu)
        check["rows_differ"] = int(diff.sum())
        if flags is not None:
            check.update(flagged=int(flags.sum()), flagged_differ=int((diff & flags).sum()),
                         unflagged_differ=int((diff & ~flags).sum()))
    # attention on sampled runs of 16 consecutive query blocks (timed), per head, with the
    # oracle's own mask.  A head's setup (its Q, K, V to fp64 and into the attention order) is
    # timed apart and extrapolated by heads; the runs are extrapolated by kept pairs.
    nbq = -(-nq // bq)
    n_slabs = path.n_slabs
    rng = np.random.default_rng(np.random.SeedSequence([cfg["seed"], 98]))
    ksz = np.minimum(bk, nk - np.arange(-(-nk // bk)) * bk)
    qsz = np.minimum(bq, nq - np.arange(nbq) * bq)
    t_setup, t_attn, pairs_done, blocks_done, heads_seen = 0.0, 0.0, 0, 0, 0
    full = name in ("ar", "ar_compact")
    run = 16
    for h in rng.permutation(H):
        b = 0
        base = 0 if n_slabs == 1 else (b * H + h) * nbq
        t1 = time.perf_counter()
        qh, kh, vh = (x[w][b, :, h].double().numpy() for w in ("q", "k", "v"))
        if perm is not None:
            qh, kh, vh = qh[perm], kh[perm], vh[perm]
        t_setup += time.perf_counter() - t1
        heads_seen += 1
        starts = np.arange(0, nbq, run)
        for c0 in (starts if full else rng.permutation(starts)):
            c1 = min(nbq, c0 + run)
            sub_rp = (rp[base + c0:base + c1 + 1] - rp[base + c0]).astype(np.int64)
            sub_ci = ci[rp[base + c0]:rp[base + c1]]
            q0, q1 = c0 * bq, min(nq, c1 * bq)
            t1 = time.perf_counter()
            o, _ = oracle.attention(qh[None, q0:q1, None], kh[None, :, None], vh[None, :, None], sub_rp, sub_ci,
                                    bq, bk, scale, 1)
            if perm is not None:                                       # the output rows back to raster order
                o_r = np.empty((q1 - q0, D))
                o_r[np.argsort(perm[q0:q1])] = o[0, :, 0]
            t_attn += time.perf_counter() - t1
            for i in range(c0, c1):
                pairs_done += int(qsz[i]) * int(ksz[ci[rp[base + i]:rp[base + i + 1]]].sum())
            blocks_done += c1 - c0
            if not full and t_attn + t_setup > target_s:
                break
        if not full and t_attn + t_setup > target_s:
            break
    pairs_total = flops_total / (4.0 * D)
    t_est = t_mask + t_setup * B * H / heads_seen + t_attn * pairs_total / max(pairs_done, 1)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    extrapolated = pairs_done < pairs_total
    return {"value": flops_total / t_est / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "extrapolated": bool(extrapolated), "t_mask_s": round(t_mask, 3), "t_head_setup_s": round(t_setup, 3),
            "t_attn_sample_s": round(t_attn, 3),
            "t_path_s": round(t_est, 3), "mask_check": check,
            "sample": (f"fp64 numpy oracle: the full mask ({'with the tile reorder of Q and K it reads, ' if dyn and perm is not None else ''}"
                       f"{t_mask:.1f} s), then attention on {blocks_done} of {B * H * nbq} (head, query block) "
                       f"pairs in runs of {run} from {heads_seen} heads ({t_attn:.1f} s, output rows reordered back; "
                       f"{t_setup:.1f} s for the heads' inputs to fp64{' and tile order' if perm is not None else ''}), "
                       + ("extrapolated to the whole path (runs by kept key-query pairs, setup by heads); "
                          if extrapolated else "")
                       + f"host has {len(os.sched_getaffinity(0))} cores available")}


def time_hbm_pass(fn, stream, flush, reps=10):
    """Median and minimum of `reps` HIP-event timings of fn on `stream`, each after reading
    the flush buffer (written once; larger than the 256 MB Infinity Cache and the L2s), so
    that every rep reads its input from HBM.  A read leaves clean lines behind: writing the
    buffer before each rep would leave dirty lines that drain during the timed call."""
    fn()
    ms = []
    for _ in range(reps):
        flush.amax()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        ms.append(a.elapsed_time(b))
    return float(np.median(ms)), float(np.min(ms))


class Path:
    """Device buffers and the calls of one workload's path (no allocation per step)."""

    def __init__(self, name, cfg, x, dev, unfused=False):
        import block_sparse_attention_masks_amd as vsa
        self.vsa, self.name, self.dev = vsa, name, dev
        # STA masks read no token data, so the step runs on raster-order tokens with the
        # tile reorder folded into the attention kernel (vsa_tiled_attn_fwd)
        self.fused = name in ("sta", "sta_heads") and not unfused
        B, H, D = cfg["batch"], cfg["heads"], cfg["head_dim"]
        self.B, self.H, self.D = B, H, D
        self.q, self.k, self.v = (x[w].to(dev) for w in ("q", "k", "v"))
        self.nq, self.nk = self.q.shape[1], self.k.shape[1]
        self.scale = D ** -0.5
        self.tiled = None
        if name in ("sta", "nabla", "nabla_sta", "sta_heads"):
            self.tiled = (cfg["grid"], cfg["tile"])
            t = cfg["tile"]
            self.bq = self.bk = t[0] * t[1] * t[2]
            self.qa, self.ka, self.va, self.oa = (torch.empty_like(self.q) for _ in range(4))
        else:
            self.bq = self.bk = cfg["block"]
            self.qa, self.ka, self.va = self.q, self.k, self.v
            self.oa = torch.empty_like(self.q)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((B, H, self.nq), dtype=torch.float32, device=dev)
        nbq, nbk = -(-self.nq // self.bq), -(-self.nk // self.bk)
        self.nbq, self.nbk = nbq, nbk
        self.n_slabs = 1 if name in ("sta", "radial") else B * H
        rows = self.n_slabs * nbq
        self.rp = torch.empty(rows + 1, dtype=torch.int32, device=dev)
        if name == "sta":
            cap = vsa.sta_capacity(cfg["grid"], cfg["tile"], cfg["window"])
            self.mask = lambda: vsa.vsa_mask_sta(cfg["grid"], cfg["tile"], cfg["window"], dev,
                                                 row_ptr=self.rp, col_idx=self.ci)
        elif name == "sta_heads":
            wins = [cfg["windows"][h % len(cfg["windows"])] for h in range(H)]
            cap = vsa.sta_heads_capacity(cfg["grid"], cfg["tile"], wins, B)
            self.mask = lambda: vsa.vsa_mask_sta_heads(cfg["grid"], cfg["tile"], wins, dev, batch=B,
                                                       row_ptr=self.rp, col_idx=self.ci)
        elif name == "radial":
            T, Hg, Wg = cfg["grid"]
            cap = nbq * nbk
            self.mask = lambda: vsa.vsa_mask_radial(T, Hg * Wg, self.bq, dev, row_ptr=self.rp,
                                                    col_idx=self.ci)
        else:
            cap = rows * nbk
            if name in ("nabla", "nabla_sta"):
                sel = dict(threshold=cfg["threshold"])
            else:
                T, Hg, Wg = cfg["grid"]
                forced = vsa.ar_forced_ranges(Hg * Wg, T, cfg["anchor_frames"], cfg["recent_frames"],
                                              self.bk)
                sel = dict(topk=cfg["topk"], forced=forced)
            ws = torch.empty(vsa.nabla_workspace_bytes(self.qa, self.ka, self.bq, self.bk, self.scale,
                                                       sel.get("threshold", 1.0), sel.get("topk", 0),
                                                       sel.get("forced", ())),
                             dtype=torch.uint8, device=dev)
            if name == "nabla_sta":
                # NABLA into scratch CSR buffers, then the union with the shared STA window
                self.rp_n = torch.empty(rows + 1, dtype=torch.int32, device=dev)
                self.ci_n = torch.empty(rows * nbk, dtype=torch.int32, device=dev)
                rp_s, ci_s = vsa.vsa_mask_sta(cfg["grid"], cfg["tile"], cfg["window"], dev)

                def mask():
                    vsa.vsa_mask_nabla(self.qa, self.ka, self.bq, self.bk, self.scale, workspace=ws,
                                       row_ptr=self.rp_n, col_idx=self.ci_n, **sel)
                    vsa.vsa_mask_union(self.rp_n, self.ci_n, B * H, rp_s, ci_s, 1, nbq, nbk,
                                       row_ptr=self.rp, col_idx=self.ci)
                self.mask = mask
            else:
                self.mask = lambda: vsa.vsa_mask_nabla(self.qa, self.ka, self.bq, self.bk, self.scale,
                                                       workspace=ws, row_ptr=self.rp, col_idx=self.ci,
                                                       **sel)
        self.ci = torch.empty(cap, dtype=torch.int32, device=dev)
        # radial: query blocks at the same place of consecutive frames share a workgroup
        # (vsa_radial_attn_fwd); the other untiled workloads group consecutive blocks
        self.frame_tokens = cfg["grid"][1] * cfg["grid"][2] if name == "radial" else None
        # workspace of the forward (union lists when small query blocks run grouped), sized
        # once: the step allocates nothing
        if self.frame_tokens:
            nws = vsa.attn_fwd_workspace_bytes_radial(self.qa, self.ka, self.rp, self.ci, self.bq, self.frame_tokens,
                                                      self.n_slabs)
        else:
            nws = vsa.attn_fwd_workspace_bytes(self.qa, self.ka, self.rp, self.ci, self.bq, self.bk, self.n_slabs)
        if self.fused:
            nws = max(nws, vsa.tiled_attn_workspace_bytes(self.q, *self.tiled, self.rp, self.ci, self.n_slabs))
        self.ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
        self.compact = None
        if name == "ar_compact":
            # size the compact cache once (the inputs are fixed); the step itself allocates nothing
            self.mask()
            slot, info = vsa.vsa_kv_plan(self.rp, self.ci, self.n_slabs, nbq, self.nk, self.bk)
            self.n_out = vsa.compact_tokens(info[:2].cpu().tolist(), self.nk, self.bk)
            self.slot, self.info = slot, info
            self.kc = torch.empty((B, self.n_out, H, D), dtype=self.k.dtype, device=dev)
            self.vc = torch.empty_like(self.kc)
            self.cc = torch.empty_like(self.ci)

            def compact():
                vsa.vsa_kv_plan(self.rp, self.ci, self.n_slabs, nbq, self.nk, self.bk, slot=self.slot, info=self.info)
                vsa.vsa_kv_gather(self.k, self.slot, self.n_slabs, self.bk, self.n_out, out=self.kc)
                vsa.vsa_kv_gather(self.v, self.slot, self.n_slabs, self.bk, self.n_out, out=self.vc)
                vsa.vsa_mask_remap(self.rp, self.ci, self.n_slabs, nbq, self.slot, nbk, out=self.cc)
            self.compact = compact

    def stages(self):
        if self.fused:
            return [("mask", self.mask), ("attn", self.attn)]
        out = [("reorder_in", self.reorder_in), ("mask", self.mask)]
        if self.compact is not None:
            out.append(("compact", self.compact))
        return out + [("attn", self.attn), ("reorder_out", self.reorder_out)]

    def reorder_in(self):
        if self.tiled:
            for src, dst in ((self.q, self.qa), (self.k, self.ka), (self.v, self.va)):
                self.vsa.vsa_tile_reorder(src, *self.tiled, out=dst)

    def attn(self, rp=None, ci=None, ws=None):
        if self.fused:   # raster q, k, v -> raster o and lse
            wsx = self.ws if rp is None else ws
            self.vsa.vsa_tiled_attn_fwd(self.q, self.k, self.v, *self.tiled, self.rp if rp is None else rp,
                                        self.ci if ci is None else ci, self.n_slabs if rp is None else 1,
                                        self.scale, out=self.o, lse=self.lse, workspace=wsx,
                                        grouped=wsx is not None)
            return
        self.attn_tile_order(rp, ci, ws)

    def attn_tile_order(self, rp=None, ci=None, ws=None):
        """The forward on the attention-order (tile-major) tensors qa, ka, va -> oa, lse."""
        if rp is None and self.compact is not None:   # over the compact cache
            self.vsa.vsa_block_sparse_attn_fwd(self.qa, self.kc, self.vc, self.rp, self.cc, self.bq, self.bk,
                                               self.n_slabs, self.scale, out=self.oa, lse=self.lse,
                                               workspace=self.ws, grouped=self.ws is not None)
            return
        wsx = self.ws if rp is None else ws
        self.vsa.vsa_block_sparse_attn_fwd(self.qa, self.ka, self.va, self.rp if rp is None else rp,
                                           self.ci if ci is None else ci, self.bq, self.bk,
                                           self.n_slabs if rp is None else 1, self.scale,
                                           out=self.oa, lse=self.lse, workspace=wsx, grouped=wsx is not None,
                                           frame_tokens=self.frame_tokens)

    def reorder_out(self):
        if self.tiled:
            self.vsa.vsa_tile_reorder(self.oa, *self.tiled, inverse=True, out=self.o)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="radial", choices=sorted(DESCRIPTION))
    ap.add_argument("--dense-reps", type=int, default=3)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--clock-s", type=float, default=1.5,
                    help="seconds of back-to-back attention calls over which the GFX clock is sampled")
    ap.add_argument("--unfused", action="store_true",
                    help="sta / sta_heads: run the tile reorder as its own passes around the attention")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the path would shard by "
              "head with no communication, and no multi-GPU run is implemented.", file=sys.stderr)
        sys.exit(2)

    from workloads import gen
    from workloads.configs import CONFIGS

    name = args.workload
    cfg = CONFIGS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    x = gen.make_inputs(name)
    print(f"[bench] {name}: inputs generated in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)
    path = Path(name, cfg, x, dev, unfused=args.unfused)
    stream = torch.cuda.current_stream(dev)
    stage_fns = path.stages()
    stages = tuple(n_ for n_, _ in stage_fns)
    ev = {s: [] for s in stages}

    def step(record):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(stage_fns) + 1)] if record else None
        for i, (_, fn) in enumerate(stage_fns):
            if record:
                marks[i].record(stream)
            fn()
        if record:
            marks[-1].record(stream)
        return marks

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    all_marks = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        all_marks.append(step(True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    for m in all_marks:
        for i, s in enumerate(stages):
            ev[s].append(m[i].elapsed_time(m[i + 1]))
    ms_step = wall * 1e3 / args.steps

    # the clock the attention kernel runs at: sampled while it runs back to back for a while
    # (enqueued ~50 ms at a time)
    attn_fn = dict(stage_fns)["attn"]
    n_inner = max(1, min(16, int(50.0 / max(float(np.mean(ev["attn"])), 1e-3))))
    with ClockSampler() as clock:
        t_end = time.perf_counter() + args.clock_s
        while time.perf_counter() < t_end:
            for _ in range(n_inner):
                attn_fn()
            torch.cuda.synchronize()
    sclk = clock.result(f"the attention kernel ran back to back for {args.clock_s:.1f} s after the timed steps")
    print(f"[bench] GFX clock under the attention kernel: {sclk}", file=sys.stderr, flush=True)

    rp_h = path.rp.cpu().numpy()
    ci_h = path.ci[: int(rp_h[-1])].cpu().numpy()
    flops = attn_flops(rp_h, ci_h, path.bq, path.bk, path.nq, path.nk, path.D, path.B * path.H, path.n_slabs)
    attn_ms = float(np.mean(ev["attn"]))
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    print(f"[bench] step {ms_step:.3f} ms; per-stage ms: " +
          ", ".join(f"{k_}={np.mean(v_):.3f}" for k_, v_ in ev.items()), file=sys.stderr, flush=True)

    dense = None
    if not args.no_dense:
        drp, dci = path.vsa.all_ones_mask(path.nbq, path.nbk, dev)
        nwd = (path.vsa.tiled_attn_workspace_bytes(path.q, *path.tiled, drp, dci, 1) if path.fused else
               path.vsa.attn_fwd_workspace_bytes_radial(path.qa, path.ka, drp, dci, path.bq, path.frame_tokens, 1)
               if path.frame_tokens else
               path.vsa.attn_fwd_workspace_bytes(path.qa, path.ka, drp, dci, path.bq, path.bk, 1))
        dws = torch.empty(nwd, dtype=torch.uint8, device=dev) if nwd else None
        path.attn(drp, dci, dws)
        dms = []
        for _ in range(args.dense_reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            path.attn(drp, dci, dws)
            b.record(stream)
            b.synchronize()
            dms.append(a.elapsed_time(b))
        dense_flops = 4.0 * path.D * path.nq * path.nk * path.B * path.H
        dense = {"ms": float(np.mean(dms)), "tflops": dense_flops / (np.mean(dms) * 1e-3) / 1e12,
                 "speedup_vs_dense": float(np.mean(dms)) / attn_ms}
        print(f"[bench] dense run {dense['ms']:.2f} ms ({dense['tflops']:.1f} TFLOP/s)", file=sys.stderr, flush=True)

    # Backward over the same mask (gradients of sum(dO * O)), timed on its own after the
    # forward, with a seeded dO.  FLOPs are counted as 2.5x the forward's kept-block FLOPs
    # (the five products S, dP, dV, dQ, dK); recomputing S and dP in both kernels is not counted.
    if path.fused:   # the backward and SICS legs take the attention-order (tile-major) tensors
        path.reorder_in()
    bwd = None
    if not args.no_bwd:
        kx, vx, cx = ((path.kc, path.vc, path.cc) if path.compact is not None else (path.ka, path.va, path.ci))
        gd = torch.Generator(device=dev).manual_seed(7)
        dout = torch.randn(path.oa.shape, generator=gd, device=dev).to(path.oa.dtype)
        path.attn_tile_order()
        dq_, dk_, dv_ = (torch.empty(t.shape, dtype=torch.float32, device=dev) for t in (path.qa, kx, vx))
        bargs = (path.qa, kx, vx, path.oa, dout, path.lse, path.rp, cx, path.bq, path.bk, path.n_slabs, path.scale)
        wsb = torch.empty(max(1, path.vsa.attn_bwd_workspace_bytes(*bargs)), dtype=torch.uint8, device=dev)
        bms = []
        for rep_ in range(4):                                  # the first call is a warm-up
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            path.vsa.vsa_block_sparse_attn_bwd(*bargs, dq=dq_, dk=dk_, dv=dv_, workspace=wsb)
            b.record(stream)
            b.synchronize()
            if rep_:
                bms.append(a.elapsed_time(b))
        bwd_ms = float(np.mean(bms))
        bwd = {"ms": round(bwd_ms, 4), "tflops": round(2.5 * flops / (bwd_ms * 1e-3) / 1e12, 2),
               "pct_bf16_peak": round(100 * 2.5 * flops / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
               "flops_counted": 2.5 * flops, "outputs": "dq, dk, dv fp32"}
        print(f"[bench] backward {bwd_ms:.3f} ms ({bwd['tflops']:.1f} TFLOP/s at 2.5x forward FLOPs)",
              file=sys.stderr, flush=True)

    # HBM-bound passes, each timed on its own outside the step with the caches flushed
    # before every rep (median and minimum of the reps), against the HBM peak:
    #   SICS block scores (SPADE's scheme-step score) of the attention-order K;
    #   the block mean-pool of the NABLA mask (its first pass), over the same K;
    #   the tile reorder of one token tensor, where the path has tiles.
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)     # 1 GiB
    k_bytes = path.ka.numel() * path.ka.element_size()

    def hbm(ms_med, ms_min, nbytes, **extra):
        gbs = nbytes / (ms_med * 1e-3) / 1e9
        return {"ms_median": round(ms_med, 4), "ms_min": round(ms_min, 4), "bytes": nbytes, "gbs": round(gbs, 1),
                "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                "frac_hbm_at_min": round(nbytes / (ms_min * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), **extra}

    sics_out = torch.empty((path.B, path.H, path.nbk), dtype=torch.float64, device=dev)
    med, mn = time_hbm_pass(lambda: path.vsa.vsa_block_sics(path.ka, path.bk, out=sics_out), stream, flush)
    sics = hbm(med, mn, k_bytes, kernel="sics_kernel", tensor="K in attention order", block=path.bk,
               ratio_to_attn=round(med / attn_ms, 5))
    pool_out = torch.empty((path.B, path.nbk, path.H, path.D), dtype=torch.float64, device=dev)
    med, mn = time_hbm_pass(lambda: path.vsa.vsa_block_mean_pool(path.ka, path.bk, out=pool_out), stream, flush)
    pool = hbm(med, mn, k_bytes, kernel="pool_kernel<true>",
               tensor="K in attention order", block=path.bk,
               bytes_written=pool_out.numel() * 8,
               gbs_with_writes=round((k_bytes + pool_out.numel() * 8) / (med * 1e-3) / 1e9, 1))
    reorder = None
    if path.tiled:
        med, mn = time_hbm_pass(lambda: path.vsa.vsa_tile_reorder(path.k, *path.tiled, out=path.ka), stream, flush)
        reorder = hbm(med, mn, 2 * k_bytes, kernel="tile_reorder_kernel", tensor="K, raster -> tile-major")
    del flush
    for nm, r in (("SICS", sics), ("pool", pool), ("reorder", reorder)):
        if r is not None:
            print(f"[bench] {nm}: median {r['ms_median']:.3f} ms (min {r['ms_min']:.3f}), {r['gbs']:.0f} GB/s "
                  f"({100 * r['frac_hbm']:.1f}% of HBM; {100 * r['frac_hbm_at_min']:.1f}% at the minimum)",
                  file=sys.stderr, flush=True)

    traffic = None
    if os.path.exists(TRAFFIC_FILE.format(name)):
        with open(TRAFFIC_FILE.format(name)) as f:
            tr = json.load(f)
        if tr.get("attn_src_sha256_16") == source_hash(ATTN_SRC):
            traffic = tr.get("bytes_per_launch")

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(name, cfg, x, path, rp_h, ci_h, flops)
        print(f"[bench] cpu baseline {cpu['value']:.4f} TFLOP/s ({cpu['sample']}); mask check {cpu['mask_check']}",
              file=sys.stderr, flush=True)

    token_bytes = path.q.numel() * path.q.element_size()
    reorder_ms = (float(np.mean(ev["reorder_in"]) + np.mean(ev["reorder_out"])) if "reorder_in" in ev else None)
    out = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DESCRIPTION[name], "global_batch": path.B, "seq_len": path.nq,
                   "kv_len": path.nk, "heads": path.H, "head_dim": path.D, "block": path.bq,
                   "mask_slabs": path.n_slabs, "kept_block_pairs": int(len(ci_h)),
                   "kept_fraction": round(len(ci_h) / (path.n_slabs * path.nbq * path.nbk), 5),
                   "parallelism": "none (one GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": attn_kernel_name(path.D, path.bq, path.bk, path.ws is not None,
                                                                 path.B, path.H, path.nbq, path.fused, path.nbk,
                                                                 path.nq, path.nk),
                     "flops_per_launch": flops, "ms_per_launch": round(attn_ms, 4),
                     # the same fraction against the peak scaled to the mean clock sampled in
                     # the timed steps (the published peak assumes 2.4 GHz)
                     "frac_at_measured_sclk": (None if sclk["mean_mhz"] is None else round(
                         attn_tflops / (PEAK_BF16_TFLOPS * sclk["mean_mhz"] / ClockSampler.SPEC_MHZ), 4))},
        "sclk": sclk,
        "cpu_baseline": cpu,
        "attn_tflops": round(attn_tflops, 2),
        "attn_pct_bf16_peak": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
        "speedup_vs_dense": None if dense is None else round(dense["speedup_vs_dense"], 3),
        "dense_ms": None if dense is None else round(dense["ms"], 3),
        "dense_tflops": None if dense is None else round(dense["tflops"], 2),
        "stage_ms": {k_: round(float(np.mean(v_)), 4) for k_, v_ in ev.items()},
        "hbm_passes": {"sics": sics, "pool": pool, "tile_reorder": reorder,
                       "method": "HIP events around each call, the caches flushed (a 1 GiB buffer read) before "
                                 "each of 10 reps; GB/s from the median"},
        "backward": bwd,
        "kv_compaction": (None if path.compact is None else
                          {"tokens_before": path.nk, "tokens_after": path.n_out,
                           "reduction": round(1 - path.n_out / path.nk, 4),
                           "ms": round(float(np.mean(ev["compact"])), 4),
                           "bytes_moved": 2 * 2 * path.B * path.n_out * path.H * path.D * path.k.element_size()}),
        "mask_over_attn": round(float(np.mean(ev["mask"])) / attn_ms, 5),
        "reorder_in_step_gbs": (round(4 * 2 * token_bytes / (reorder_ms * 1e-3) / 1e9, 1)
                                if path.tiled and reorder_ms else None),
        "tile_reorder": (None if not path.tiled else
                         "folded into the attention kernel (raster-order q, k, v, o)" if path.fused else
                         "separate passes: q, k, v in, o out"),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

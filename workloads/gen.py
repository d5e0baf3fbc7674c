"""Seeded synthetic inputs shared by the fp64 oracle and the GPU path.

This module holds no arithmetic of the method (no reorder, mask or attention);
it only draws numbers.  Recipe:

* Random streams: numpy ``default_rng(SeedSequence([seed, stream, b, h, chunk]))``
  with stream 1 = Q noise, 2 = K noise, 3 = V noise, and tokens cut into chunks of
  65,536; the frequencies use ``SeedSequence([seed, 0])``.  Every (tensor, batch,
  head, chunk) is therefore independent of every other and can be regenerated on
  its own -- the oracle rebuilds one head of a 450,000-token tensor without
  building the rest.
* Values: ``x = noise * N(0,1) + P`` where P (when the workload has one) is the
  per-head positional code 1.5*cos(w_j . x_tok) for feature j < D/2 and
  1.5*sin(w_{j-D/2} . x_tok) for j >= D/2, x_tok = integer raster coordinates
  (t, h, w) of the token, w_j ~ U[-0.6, 0.6]^3 drawn per (head, j).
* Rounding: fp64 -> fp32 (round to nearest even) -> bf16 (round to nearest even)
  once, for bf16 workloads.  The rounded tensor is the single source of truth: the
  oracle reads it upcast to fp64, the GPU reads it as is.

Layout of every token tensor: [batch, tokens, heads, head_dim], head_dim fastest,
tokens in raster order (t, h, w), w fastest.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from .configs import CONFIGS, n_tokens, q_grid, q_frame_offset

CHUNK = 65536
STREAM = {"q": 1, "k": 2, "v": 3}
_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def _cfg(cfg):
    return CONFIGS[cfg] if isinstance(cfg, str) else cfg


def omega(cfg):
    """Frequency vectors [heads, head_dim // 2, 3], fp64, U[-0.6, 0.6]."""
    cfg = _cfg(cfg)
    rng = np.random.default_rng(np.random.SeedSequence([cfg["seed"], 0]))
    return rng.uniform(-0.6, 0.6, size=(cfg["heads"], cfg["head_dim"] // 2, 3))


def token_coords(grid, lo, hi, t0=0):
    """Integer raster coordinates (t, h, w) of tokens [lo, hi) of a T x H x W grid."""
    _, hh, ww = grid
    n = np.arange(lo, hi, dtype=np.int64)
    return np.stack([n // (hh * ww) + t0, (n // ww) % hh, n % ww], axis=1).astype(np.float64)


def _tensor_grid(cfg, which):
    if which == "q":
        return q_grid(cfg), q_frame_offset(cfg)
    return cfg["grid"], 0


def _values(cfg, which, b, h, lo, hi, om):
    """Unrounded fp64 values of tokens [lo, hi) of one (batch, head): [hi-lo, D]."""
    d = cfg["head_dim"]
    grid, t0 = _tensor_grid(cfg, which)
    out = np.empty((hi - lo, d), dtype=np.float64)
    c0 = lo // CHUNK
    c1 = (hi - 1) // CHUNK
    for c in range(c0, c1 + 1):
        clo, chi = c * CHUNK, min((c + 1) * CHUNK, n_tokens(grid))
        rng = np.random.default_rng(
            np.random.SeedSequence([cfg["seed"], STREAM[which], b, h, c]))
        z = rng.standard_normal((chi - clo, d))
        a, e = max(lo, clo), min(hi, chi)
        out[a - lo:e - lo] = z[a - clo:e - clo]
    noise = 1.0 if which == "v" else cfg["qk_noise"]
    if noise != 1.0:
        out *= noise
    use_pos = cfg["positional"] if which in ("q", "k") else cfg["v_positional"]
    if use_pos:
        ang = token_coords(grid, lo, hi, t0) @ om[h].T          # [n, D/2]
        out[:, : d // 2] += 1.5 * np.cos(ang)
        out[:, d // 2:] += 1.5 * np.sin(ang)
    return out


def _round(x64, dtype):
    """fp64 numpy -> torch tensor of the workload dtype (fp32 RNE, then bf16 RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))
    return t.to(_TORCH_DTYPE[dtype]) if dtype != "f32" else t


def tokens(cfg, which):
    cfg = _cfg(cfg)
    return n_tokens(_tensor_grid(cfg, which)[0])


def head_values(cfg, which, b, h, lo=0, hi=None):
    """Rounded values of one (batch, head) as fp64 numpy [hi-lo, D].

    Bit-identical to ``make_tensor(cfg, which)[b, lo:hi, h, :]`` upcast to fp64."""
    cfg = _cfg(cfg)
    hi = tokens(cfg, which) if hi is None else hi
    x = _values(cfg, which, b, h, lo, hi, omega(cfg))
    return _round(x, cfg["dtype"]).to(torch.float64).numpy()


def make_tensor(cfg, which, threads=None):
    """Full rounded tensor [batch, tokens, heads, head_dim] (torch, CPU)."""
    cfg = _cfg(cfg)
    bsz, nh, d = cfg["batch"], cfg["heads"], cfg["head_dim"]
    n = tokens(cfg, which)
    om = omega(cfg)
    out = torch.empty((bsz, n, nh, d), dtype=_TORCH_DTYPE[cfg["dtype"]])
    threads = threads or min(16, len(os.sched_getaffinity(0)))

    def task(bh):
        b, h = bh
        for lo in range(0, n, CHUNK):
            hi = min(n, lo + CHUNK)
            out[b, lo:hi, h, :] = _round(_values(cfg, which, b, h, lo, hi, om), cfg["dtype"])

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(task, [(b, h) for b in range(bsz) for h in range(nh)]))
    return out


def make_inputs(cfg, threads=None):
    """dict(q=..., k=..., v=...) of rounded CPU tensors for a workload."""
    return {w: make_tensor(cfg, w, threads) for w in ("q", "k", "v")}


def sample_rows(cfg, n_rows, seed_tag=99):
    """Uniform sample (without replacement) of (batch, head, query token) output rows.

    Always includes the last query token (the ragged tail) of head 0."""
    cfg = _cfg(cfg)
    nq = tokens(cfg, "q")
    total = cfg["batch"] * cfg["heads"] * nq
    rng = np.random.default_rng(np.random.SeedSequence([cfg["seed"], seed_tag]))
    idx = rng.choice(total, size=min(n_rows, total), replace=False)
    last = nq - 1
    if last not in idx:
        idx[0] = last
    idx = np.sort(idx)
    b = idx // (cfg["heads"] * nq)
    h = (idx // nq) % cfg["heads"]
    t = idx % nq
    return np.stack([b, h, t], axis=1)

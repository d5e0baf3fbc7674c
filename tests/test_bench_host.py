"""Host-side logic of bench.py (no GPU): the algorithmic FLOP count behind the headline
metric, the label of the attention kernel whose launches the roofline divides by, the
one-GPU refusal and the clock sampler's failure path."""
import os
import subprocess
import sys
import time

import numpy as np
import pytest

import bench
from oracle.masks import csr_from_bool

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _flops_by_pairs(keep, block_q, block_k, nq, nk, D, slab_mult):
    """4 D times the token pairs of every kept block pair, counted pair by pair."""
    total = 0
    for r in range(keep.shape[0]):
        i = r % (-(-nq // block_q))
        nqi = min(block_q, nq - i * block_q)
        for j in np.flatnonzero(keep[r]):
            total += nqi * min(block_k, nk - j * block_k)
    return 4.0 * D * total * slab_mult


@pytest.mark.parametrize("nq,nk,bq,bk,slabs,bh", [
    (300, 250, 64, 48, 1, 6),    # ragged last blocks on both sides, one shared mask for 6 heads
    (256, 256, 64, 64, 3, 3),    # one mask per head, no tails
    (130, 1000, 64, 64, 2, 2),   # two-token query tail, eight-token key tail
])
def test_attn_flops_counts_every_token_pair(nq, nk, bq, bk, slabs, bh):
    rng = np.random.default_rng(7)
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    keep = rng.random((slabs * nbq, nbk)) < 0.4
    keep[:, -1] |= rng.random(slabs * nbq) < 0.5       # the ragged key block kept by some rows
    keep[1] = False                                      # an empty row
    rp, ci = csr_from_bool(keep)
    got = bench.attn_flops(rp, ci, bq, bk, nq, nk, 128, bh, slabs)
    want = _flops_by_pairs(keep, bq, bk, nq, nk, 128, bh if slabs == 1 else 1)
    assert got == want


def test_attn_flops_dense_closed_form():
    # all blocks kept: 4 D nq nk per (b, h), whatever the block sizes and tails
    nq, nk, bq, bk = 1000, 777, 128, 64
    keep = np.ones((-(-nq // bq), -(-nk // bk)), dtype=bool)
    rp, ci = csr_from_bool(keep)
    assert bench.attn_flops(rp, ci, bq, bk, nq, nk, 64, 5, 1) == 4.0 * 64 * nq * nk * 5


@pytest.mark.parametrize("profile,args", [
    ("path_sta_kernel_stats.md", dict(D=128, block_q=384, block_k=384, grouped=True, heads=24,
                                      n_qblocks=300, tiled=True, nq=115200, nk=115200)),
    ("path_nabla_kernel_stats.md", dict(D=128, block_q=64, block_k=64, grouped=True, heads=40,
                                        n_qblocks=960, nq=61440, nk=61440)),
    ("path_radial_kernel_stats.md", dict(D=128, block_q=128, block_k=128, grouped=True, heads=24,
                                         n_qblocks=3516, nq=450000, nk=450000)),
    ("path_ar_kernel_stats.md", dict(D=128, block_q=64, block_k=64, grouped=True, heads=12,
                                     n_qblocks=74, n_kblocks=512, nq=4680, nk=32760)),
])
def test_kernel_label_is_the_profiled_kernel(profile, args):
    """The label the bench line divides by must name the kernel the trace of that
    workload shows as its attention launch."""
    name = bench.attn_kernel_name(**args)
    with open(os.path.join(ROOT, "profiles", profile)) as f:
        rows = [line for line in f if line.startswith("| attn_fwd_bf16_kernel")]
    assert rows, profile
    assert any(line.split("|")[1].strip() == name for line in rows), (name, rows)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_clock_sampler_reports_instead_of_failing():
    t0 = time.monotonic()
    with bench.ClockSampler(interval_s=0.01) as c:
        time.sleep(0.05)
    assert time.monotonic() - t0 < 10.0
    r = c.result("a test")
    if r["mean_mhz"] is None:          # no driver or no permission: a reason, not an exception
        assert isinstance(r["error"], str) and r["error"]
    else:
        assert 100.0 < r["mean_mhz"] < 5000.0 and r["samples"] >= 1

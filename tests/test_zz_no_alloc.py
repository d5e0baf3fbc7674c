"""The allocation-free forward (vsa_block_sparse_attn_fwd_static) against the forward with a
caller-supplied workspace, through the C ABI: identical bits on calls in a row that use the
library's fixed scratch array (grouped union lists, then split partial outputs), each call on
a smaller input than the one before."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_attention_masks_amd as vsa
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(nq, nk, H, bq, bk, dens, seed):
    g = torch.Generator().manual_seed(seed)
    q, k, v = (torch.randn((1, n, H, 128), generator=g).to(torch.bfloat16).to(DEV) for n in (nq, nk, nk))
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    rng = np.random.default_rng(seed)
    keep = rng.random((H * nbq, nbk)) < dens
    keep[np.arange(H * nbq), rng.integers(0, nbk, size=H * nbq)] = True
    rp, ci = oracle.csr_from_bool(keep)
    return q, k, v, torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV)


# (nq, nk, heads, block_q, block_k, density): grouped 12-wave, then grouped 8-wave on a smaller
# problem, then split key streams on a still smaller one
CASES = [(4096, 4096, 48, 64, 64, 0.4), (3000, 2500, 24, 64, 64, 0.5), (1000, 5000, 2, 64, 64, 0.3)]


def test_static_forward_matches_workspace_forward():
    sizes = []
    for i, (nq, nk, H, bq, bk, dens) in enumerate(CASES):
        print(f"static forward case {i}: nq={nq} nk={nk} heads={H} blocks {bq}/{bk}", flush=True)
        q, k, v, rp, ci = _case(nq, nk, H, bq, bk, dens, 100 + i)
        need = vsa.attn_fwd_workspace_bytes(q, k, rp, ci, bq, bk, H)
        assert 0 < need <= 64 << 20                     # this case uses the scratch array
        sizes.append(q.numel() + k.numel())
        o_ref, l_ref = vsa.vsa_block_sparse_attn_fwd(q, k, v, rp, ci, bq, bk, H)
        out = torch.full_like(q, float("nan"))
        lse = torch.full((1, H, nq), float("nan"), dtype=torch.float32, device=DEV)
        vsa.vsa_block_sparse_attn_fwd_static(q, k, v, rp, ci, bq, bk, out, lse, H)
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(lse, l_ref), i
    assert sizes[1] < sizes[0] and sizes[2] < sizes[1]


def test_static_forward_rejects_oversize_before_any_launch():
    """Union lists above 64 MiB: VSA_ERR_CAPACITY, nothing launched, out untouched."""
    H, n, b = 256, 30000, 64
    L = vsa.lib()
    fake = ctypes.c_void_p(0x1000)
    st = L.vsa_block_sparse_attn_fwd_static(fake, fake, fake, fake, None, 1, 1, H, 128, n, n, b, b, fake, fake, H,
                                            0.1, None)
    assert st == -5

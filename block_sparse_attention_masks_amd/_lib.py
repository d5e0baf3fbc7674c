"""ctypes binding of libvsa.so: argument marshalling only.

Torch tensors supply device memory and the stream; every step of the path runs
in the library's HIP kernels.  There is no CPU fallback: if the library is not
built, every call raises.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# VSA_LIB names another build of the same library (e.g. the host-sanitized one); default: in-tree
LIB_PATH = os.environ.get("VSA_LIB") or os.path.join(_PKG, "libvsa.so")

VSA_F32, VSA_BF16 = 0, 1
_DTYPE = {torch.float32: VSA_F32, torch.bfloat16: VSA_BF16}


class VsaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class Select(ctypes.Structure):
    _fields_ = [("cdf_threshold", ctypes.c_double), ("topk", ctypes.c_int32),
                ("n_forced", ctypes.c_int32), ("forced", ctypes.POINTER(ctypes.c_int32))]


_lib = None

_P, _I32, _I64, _F32, _F64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
_SIGS = {
    "vsa_status_string": ([_I32], ctypes.c_char_p),
    "vsa_tile_reorder": ([_P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I64, _I32, _P], _I32),
    "vsa_mask_sta": ([_I32] * 9 + [_P, _P, _I64, _P], _I32),
    "vsa_mask_radial": ([_I32, _I32, _I32, _P, _P, _I64, _P], _I32),
    "vsa_mask_sta_heads": ([_I32] * 6 + [_P, _I32, _I64, _P, _P, _I64, _P], _I32),
    "vsa_mask_union": ([_I64, _I32, _P, _P, _I64, _P, _P, _I64, _P, _P, _I64, _P], _I32),
    "vsa_block_sics": ([_P, _I32, _I64, _I32, _I32, _I64, _I32, _P, _P], _I32),
    "vsa_block_mean_pool": ([_P, _I32, _I64, _I32, _I32, _I64, _I32, _P, _P], _I32),
    "vsa_block_sparse_attn_bwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I64, _I64, _I32,
                                   _I32, _P, _P, _I32, _F32, _P, ctypes.POINTER(ctypes.c_size_t), _P], _I32),
    "vsa_kv_plan": ([_P, _P, _I64, _I64, _I64, _I32, _P, _P, _P], _I32),
    "vsa_kv_gather": ([_P, _I32, _I64, _I32, _I32, _I64, _I32, _P, _I64, _P, _I64, _P], _I32),
    "vsa_mask_remap": ([_P, _P, _I64, _I64, _P, _I32, _P, _P], _I32),
    "vsa_mask_nabla": ([_P, _P, _I32, _I64, _I32, _I32, _I64, _I64, _I32, _I32, _F64,
                        ctypes.POINTER(Select), _P, _P, _I64, _P, ctypes.POINTER(ctypes.c_size_t), _P], _I32),
    "vsa_block_sparse_attn_fwd": ([_P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I64, _I64, _I32, _I32,
                                   _P, _P, _I32, _F32, _P, ctypes.POINTER(ctypes.c_size_t), _P], _I32),
    "vsa_block_sparse_attn_fwd_static": ([_P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I64, _I64, _I32, _I32,
                                          _P, _P, _I32, _F32, _P], _I32),
    "vsa_radial_attn_fwd": ([_P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I64, _I64, _I32, _I32, _I64,
                             _P, _P, _I32, _F32, _P, ctypes.POINTER(ctypes.c_size_t), _P], _I32),
    "vsa_tiled_attn_fwd": ([_P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                            _P, _P, _I32, _F32, _P, ctypes.POINTER(ctypes.c_size_t), _P], _I32),
}
EXPORTS = tuple(_SIGS)


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_masks_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(h, name)
            fn.argtypes, fn.restype = args, res
        _lib = h
    return _lib


def status_string(status):
    return lib().vsa_status_string(status).decode()


def _check(status, where):
    if status != 0:
        raise VsaError(status, where)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _require(t, name, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU (no CPU path exists)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


# ----------------------------------------------------------------------------- calls
def vsa_tile_reorder(src, grid, tile, inverse=False, out=None):
    """Tile reorder of src [B, T*H*W, heads, head_dim] (any dtype); returns dst."""
    _require(src, "src")
    out = torch.empty_like(src) if out is None else out
    _require(out, "out", src.device)
    T, H, W = grid
    tt, th, tw = tile
    row_bytes = src[0, 0].numel() * src.element_size()
    _check(lib().vsa_tile_reorder(_ptr(src), _ptr(out), src.shape[0], T, H, W, tt, th, tw,
                                  row_bytes, int(bool(inverse)), _stream(src)), "vsa_tile_reorder")
    return out


def sta_capacity(grid, tile, window):
    n = [g // t for g, t in zip(grid, tile)]
    return n[0] * n[1] * n[2] * min(window[0], n[0]) * min(window[1], n[1]) * min(window[2], n[2])


def vsa_mask_sta(grid, tile, window, device, row_ptr=None, col_idx=None):
    """STA tile-window mask -> (row_ptr, col_idx) int32 device tensors.

    col_idx is allocated at the capacity the call requires; its first
    row_ptr[-1] entries are the mask.  Preallocated outputs may be passed."""
    n = (grid[0] // tile[0]) * (grid[1] // tile[1]) * (grid[2] // tile[2])
    cap = sta_capacity(grid, tile, window)
    if row_ptr is None:
        row_ptr = torch.empty(n + 1, dtype=torch.int32, device=device)
    if col_idx is None:
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=device)
    _require(row_ptr, "row_ptr")
    _require(col_idx, "col_idx", row_ptr.device)
    if row_ptr.numel() != n + 1 or row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise ValueError("row_ptr must be int32 [n_tiles + 1] and col_idx int32")
    _check(lib().vsa_mask_sta(*grid, *tile, *window, _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
                              _stream(row_ptr)), "vsa_mask_sta")
    return row_ptr, col_idx


def vsa_mask_radial(T, S, block, device, row_ptr=None, col_idx=None):
    """Radial mask over raster order -> (row_ptr, col_idx); col_idx holds
    n_blocks^2 entries, the first row_ptr[-1] of which are the mask."""
    nb = -(-(T * S) // block)
    if row_ptr is None:
        row_ptr = torch.empty(nb + 1, dtype=torch.int32, device=device)
    if col_idx is None:
        col_idx = torch.empty(nb * nb, dtype=torch.int32, device=device)
    _require(row_ptr, "row_ptr")
    _require(col_idx, "col_idx", row_ptr.device)
    if row_ptr.numel() != nb + 1 or row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise ValueError("row_ptr must be int32 [n_blocks + 1] and col_idx int32")
    _check(lib().vsa_mask_radial(T, S, block, _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
                                 _stream(row_ptr)), "vsa_mask_radial")
    return row_ptr, col_idx


def sta_heads_capacity(grid, tile, windows, batch=1):
    return batch * sum(sta_capacity(grid, tile, w) for w in windows)


def vsa_mask_sta_heads(grid, tile, windows, device, batch=1, row_ptr=None, col_idx=None):
    """STA mask with one window per head -> (row_ptr, col_idx) over batch * heads slabs
    (slab = b * heads + h); col_idx is allocated at the capacity the call requires."""
    heads = len(windows)
    n = (grid[0] // tile[0]) * (grid[1] // tile[1]) * (grid[2] // tile[2])
    cap = sta_heads_capacity(grid, tile, windows, batch)
    if row_ptr is None:
        row_ptr = torch.empty(batch * heads * n + 1, dtype=torch.int32, device=device)
    if col_idx is None:
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=device)
    _require(row_ptr, "row_ptr")
    _require(col_idx, "col_idx", row_ptr.device)
    if row_ptr.numel() != batch * heads * n + 1 or row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise ValueError("row_ptr must be int32 [batch * heads * n_tiles + 1] and col_idx int32")
    flat = [int(x) for w in windows for x in w]
    arr = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    _check(lib().vsa_mask_sta_heads(*grid, *tile, ctypes.cast(arr, ctypes.c_void_p), heads, batch,
                                    _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _stream(row_ptr)),
           "vsa_mask_sta_heads")
    return row_ptr, col_idx


def vsa_mask_union(rp_a, ci_a, slabs_a, rp_b, ci_b, slabs_b, n_qblocks, n_kblocks, row_ptr=None, col_idx=None):
    """Row-by-row union of two CSR masks (a one-slab mask is shared) -> (row_ptr, col_idx);
    col_idx is allocated at max(slabs) * n_qblocks * n_kblocks entries."""
    for t, nm in ((rp_a, "rp_a"), (ci_a, "ci_a"), (rp_b, "rp_b"), (ci_b, "ci_b")):
        _require(t, nm, rp_a.device)
        if t.dtype != torch.int32:
            raise ValueError(f"{nm} must be int32")
    slabs = max(slabs_a, slabs_b)
    rows = slabs * n_qblocks
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=rp_a.device)
    if col_idx is None:
        col_idx = torch.empty(max(1, rows * n_kblocks), dtype=torch.int32, device=rp_a.device)
    _require(row_ptr, "row_ptr", rp_a.device)
    _require(col_idx, "col_idx", rp_a.device)
    if rp_a.numel() != slabs_a * n_qblocks + 1 or rp_b.numel() != slabs_b * n_qblocks + 1:
        raise ValueError("row_ptr inputs must hold slabs * n_qblocks + 1 entries")
    if row_ptr.numel() != rows + 1 or row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise ValueError("row_ptr must be int32 [max(slabs) * n_qblocks + 1] and col_idx int32")
    _check(lib().vsa_mask_union(n_qblocks, n_kblocks, _ptr(rp_a), _ptr(ci_a), slabs_a, _ptr(rp_b), _ptr(ci_b),
                                slabs_b, _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _stream(row_ptr)),
           "vsa_mask_union")
    return row_ptr, col_idx


def vsa_block_mean_pool(x, block, out=None):
    """Mean of each block's valid token rows of x [B, N, heads, head_dim] (bf16 or fp32)
    -> fp64 [B, ceil(N / block), heads, head_dim] (block-major, like x)."""
    _require(x, "x")
    if x.dtype not in _DTYPE:
        raise ValueError("x must be bfloat16 or float32")
    B, N, H, D = x.shape
    nb = -(-N // block)
    if out is None:
        out = torch.empty((B, nb, H, D), dtype=torch.float64, device=x.device)
    _require(out, "out", x.device)
    if out.dtype != torch.float64 or tuple(out.shape) != (B, nb, H, D):
        raise ValueError("out must be float64 [B, n_blocks, heads, head_dim]")
    _check(lib().vsa_block_mean_pool(_ptr(x), _DTYPE[x.dtype], B, H, D, N, block, _ptr(out), _stream(x)),
           "vsa_block_mean_pool")
    return out


def vsa_block_sics(x, block, out=None):
    """SICS block scores of x [B, N, heads, head_dim] (bf16 or fp32) -> fp64 [B, heads, ceil(N / block)]."""
    _require(x, "x")
    if x.dtype not in _DTYPE:
        raise ValueError("x must be float32 or bfloat16")
    B, N, H, D = x.shape
    nb = -(-N // block)
    out = torch.empty((B, H, nb), dtype=torch.float64, device=x.device) if out is None else out
    _require(out, "out", x.device)
    if out.dtype != torch.float64 or tuple(out.shape) != (B, H, nb):
        raise ValueError("out must be float64 [B, heads, n_blocks]")
    _check(lib().vsa_block_sics(_ptr(x), _DTYPE[x.dtype], B, H, D, N, block, _ptr(out), _stream(x)),
           "vsa_block_sics")
    return out


def vsa_kv_plan(row_ptr, col_idx, n_slabs, n_qblocks, nk, block_k, slot=None, info=None):
    """Slot map of each mask slab -> (slot int32 [n_slabs, n_kblocks], info int32 [2 + 2 n_slabs])."""
    _require(row_ptr, "row_ptr")
    _require(col_idx, "col_idx", row_ptr.device)
    nbk = -(-nk // block_k)
    if slot is None:
        slot = torch.empty((n_slabs, nbk), dtype=torch.int32, device=row_ptr.device)
    if info is None:
        info = torch.empty(2 + 2 * n_slabs, dtype=torch.int32, device=row_ptr.device)
    _require(slot, "slot", row_ptr.device)
    _require(info, "info", row_ptr.device)
    if slot.numel() != n_slabs * nbk or info.numel() != 2 + 2 * n_slabs:
        raise ValueError("slot must hold n_slabs * n_kblocks ints and info 2 + 2 * n_slabs")
    if row_ptr.numel() != n_slabs * n_qblocks + 1:
        raise ValueError("row_ptr must hold n_slabs * n_qblocks + 1 entries")
    _check(lib().vsa_kv_plan(_ptr(row_ptr), _ptr(col_idx), n_slabs, n_qblocks, nk, block_k, _ptr(slot), _ptr(info),
                             _stream(row_ptr)), "vsa_kv_plan")
    return slot, info


def compact_tokens(info, nk, block_k):
    """Token count of the compact cache from the plan's info (host ints or tensor)."""
    n_full, has_tail = int(info[0]), int(info[1])
    return n_full * block_k + ((nk % block_k) if has_tail else 0)


def vsa_kv_gather(x, slot, n_slabs, block_k, n_out, out=None):
    """Kept blocks of x [B, nk, heads, head_dim] -> compact cache [B, n_out, heads, head_dim]."""
    _require(x, "x")
    if x.dtype not in _DTYPE:
        raise ValueError("x must be float32 or bfloat16")
    B, nk, H, D = x.shape
    if out is None:
        out = torch.empty((B, n_out, H, D), dtype=x.dtype, device=x.device)
    _require(out, "out", x.device)
    _require(slot, "slot", x.device)
    if out.dtype != x.dtype or tuple(out.shape) != (B, n_out, H, D):
        raise ValueError("out must match x's dtype and be [B, n_out, heads, head_dim]")
    _check(lib().vsa_kv_gather(_ptr(x), _DTYPE[x.dtype], B, H, D, nk, block_k, _ptr(slot), n_slabs, _ptr(out),
                               n_out, _stream(x)), "vsa_kv_gather")
    return out


def vsa_mask_remap(row_ptr, col_idx, n_slabs, n_qblocks, slot, n_kblocks, out=None):
    """Mask columns rewritten to compact slots (row_ptr unchanged) -> col_idx tensor."""
    _require(row_ptr, "row_ptr")
    _require(col_idx, "col_idx", row_ptr.device)
    _require(slot, "slot", row_ptr.device)
    if out is None:
        out = torch.empty_like(col_idx)
    _require(out, "out", row_ptr.device)
    _check(lib().vsa_mask_remap(_ptr(row_ptr), _ptr(col_idx), n_slabs, n_qblocks, _ptr(slot), n_kblocks, _ptr(out),
                                _stream(row_ptr)), "vsa_mask_remap")
    return out


def vsa_kv_compact(k, v, row_ptr, col_idx, n_slabs, block_q, block_k):
    """Plan, gather K and V, and rewrite the mask (one host sync to size the cache).
    Returns (k_compact, v_compact, col_idx_compact, n_out, slot, info)."""
    nq_blocks = (row_ptr.numel() - 1) // n_slabs
    nk = k.shape[1]
    slot, info = vsa_kv_plan(row_ptr, col_idx, n_slabs, nq_blocks, nk, block_k)
    n_out = compact_tokens(info[:2].cpu().tolist(), nk, block_k)
    kc = vsa_kv_gather(k, slot, n_slabs, block_k, n_out)
    vc = vsa_kv_gather(v, slot, n_slabs, block_k, n_out)
    cc = vsa_mask_remap(row_ptr, col_idx, n_slabs, nq_blocks, slot, -(-nk // block_k))
    return kc, vc, cc, n_out, slot, info


def attn_bwd_workspace_bytes(q, k, v, o, dout, lse, row_ptr, col_idx, block_q, block_k, n_slabs=1, scale=None):
    """Workspace bytes vsa_block_sparse_attn_bwd needs for these arguments (no launch)."""
    B, nq, H, D = q.shape
    scale = D ** -0.5 if scale is None else scale
    need = ctypes.c_size_t(0)
    _check(lib().vsa_block_sparse_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), None, None,
                                           None, _DTYPE[q.dtype], B, H, D, nq, k.shape[1], block_q, block_k,
                                           _ptr(row_ptr), _ptr(col_idx), n_slabs, scale, None, ctypes.byref(need),
                                           _stream(q)), "vsa_block_sparse_attn_bwd")
    return need.value


def vsa_block_sparse_attn_bwd(q, k, v, o, dout, lse, row_ptr, col_idx, block_q, block_k, n_slabs=1, scale=None,
                              dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dq, dk, dv) fp32 of L = sum(dout * o) for o = vsa_block_sparse_attn_fwd(q, k, v) with the
    same mask; o and lse are the forward's outputs.  The workspace is allocated if not given."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (lse, "lse"), (row_ptr, "row_ptr"),
                  (col_idx, "col_idx")):
        _require(t, nm, q.device)
    if q.dtype not in _DTYPE or any(t.dtype != q.dtype for t in (k, v, o, dout)):
        raise ValueError("q, k, v, o, dout must share one dtype (float32 or bfloat16)")
    if lse.dtype != torch.float32:
        raise ValueError("lse must be float32")
    B, nq, H, D = q.shape
    nk = k.shape[1]
    scale = D ** -0.5 if scale is None else scale
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device) if dv is None else dv
    for t, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _require(t, nm, q.device)
        if t.dtype != torch.float32:
            raise ValueError(f"{nm} must be float32")
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
            _DTYPE[q.dtype], B, H, D, nq, nk, block_q, block_k, _ptr(row_ptr), _ptr(col_idx), n_slabs, scale)
    need = ctypes.c_size_t(0)
    _check(lib().vsa_block_sparse_attn_bwd(*args, None, ctypes.byref(need), _stream(q)), "vsa_block_sparse_attn_bwd")
    if workspace is None:
        workspace = torch.empty(max(1, need.value), dtype=torch.uint8, device=q.device)
    _require(workspace, "workspace", q.device)
    nb = ctypes.c_size_t(workspace.numel())
    _check(lib().vsa_block_sparse_attn_bwd(*args, _ptr(workspace), ctypes.byref(nb), _stream(q)),
           "vsa_block_sparse_attn_bwd")
    return dq, dk, dv


def _select(threshold, topk, forced):
    flat = [int(x) for r in forced for x in r]
    arr = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    sel = Select(float(threshold if threshold is not None else 1.0), int(topk), len(forced),
                 ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)))
    return sel, arr


def nabla_workspace_bytes(q, k, block_q, block_k, scale=None, threshold=1.0, topk=0, forced=()):
    sel, _keep = _select(threshold, topk, forced)
    nbytes = ctypes.c_size_t(0)
    B, nq, Hh, D = q.shape
    rp = ctypes.c_void_p(16)  # never dereferenced by a size query
    _check(lib().vsa_mask_nabla(_ptr(q), _ptr(k), _DTYPE[q.dtype], B, Hh, D, nq, k.shape[1],
                                block_q, block_k, float(scale if scale is not None else D ** -0.5),
                                ctypes.byref(sel), rp, rp, 0, None, ctypes.byref(nbytes), None),
           "vsa_mask_nabla")
    return nbytes.value


def vsa_mask_nabla(q, k, block_q, block_k, scale=None, threshold=None, topk=0, forced=(),
                   workspace=None, row_ptr=None, col_idx=None):
    """NABLA (threshold) or anchor + recent + top-k (topk > 0) mask, one slab per
    (batch, head) -> (row_ptr, col_idx).  Preallocated outputs and workspace may be
    passed (see nabla_workspace_bytes)."""
    _require(q, "q")
    _require(k, "k", q.device)
    B, nq, Hh, D = q.shape
    nk = k.shape[1]
    scale = D ** -0.5 if scale is None else scale
    sel, _keep = _select(threshold, topk, forced)
    nbq, nbk = -(-nq // block_q), -(-nk // block_k)
    rows = B * Hh * nbq
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=q.device)
    if col_idx is None:
        col_idx = torch.empty(rows * nbk, dtype=torch.int32, device=q.device)
    _require(row_ptr, "row_ptr", q.device)
    _require(col_idx, "col_idx", q.device)
    if row_ptr.numel() != rows + 1 or row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise ValueError("row_ptr must be int32 [batch*heads*n_qblocks + 1] and col_idx int32")
    if workspace is None:
        need = nabla_workspace_bytes(q, k, block_q, block_k, scale, sel.cdf_threshold, topk, forced)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    _check(lib().vsa_mask_nabla(_ptr(q), _ptr(k), _DTYPE[q.dtype], B, Hh, D, nq, nk, block_q,
                                block_k, float(scale), ctypes.byref(sel), _ptr(row_ptr),
                                _ptr(col_idx), col_idx.numel(), _ptr(workspace), ctypes.byref(nbytes),
                                _stream(q)), "vsa_mask_nabla")
    return row_ptr, col_idx


def vsa_block_sparse_attn_fwd_static(q, k, v, row_ptr, col_idx, block_q, block_k, out, lse, n_slabs=1, scale=None):
    """vsa_block_sparse_attn_fwd with its workspace in the library's fixed device array:
    nothing is allocated (out and lse are the caller's).  Calls that overlap on one GPU race."""
    for name, t in (("q", q), ("k", k), ("v", v), ("row_ptr", row_ptr), ("col_idx", col_idx), ("out", out)):
        _require(t, name, q.device)
    if lse is not None:
        _require(lse, "lse", q.device)
    B, nq, Hh, D = q.shape
    scale = D ** -0.5 if scale is None else scale
    _check(lib().vsa_block_sparse_attn_fwd_static(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _DTYPE[q.dtype], B,
                                                  Hh, D, nq, k.shape[1], block_q, block_k, _ptr(row_ptr),
                                                  _ptr(col_idx), n_slabs, float(scale), _stream(q)),
           "vsa_block_sparse_attn_fwd_static")
    return out, lse


def vsa_radial_attn_fwd(q, k, v, row_ptr, col_idx, block, frame_tokens, n_slabs=1, scale=None, out=None, lse=None,
                        want_lse=True, workspace=None, grouped=True):
    """vsa_block_sparse_attn_fwd for masks over raster-order frames of frame_tokens tokens:
    with a workspace, query blocks at the same place of consecutive frames share a
    workgroup (same result; only the work order differs)."""
    return vsa_block_sparse_attn_fwd(q, k, v, row_ptr, col_idx, block, block, n_slabs, scale, out, lse, want_lse,
                                     workspace, grouped, frame_tokens=frame_tokens)


def attn_fwd_workspace_bytes_radial(q, k, row_ptr, col_idx, block, frame_tokens, n_slabs=1):
    """Workspace bytes of vsa_radial_attn_fwd (0: none)."""
    B, nq, Hh, D = q.shape
    nb = ctypes.c_size_t(0)
    _check(lib().vsa_radial_attn_fwd(_ptr(q), _ptr(k), _ptr(k), _ptr(q), None, _DTYPE[q.dtype], B, Hh, D, nq,
                                     k.shape[1], block, block, frame_tokens, _ptr(row_ptr), _ptr(col_idx), n_slabs,
                                     1.0, None, ctypes.byref(nb), None), "vsa_radial_attn_fwd")
    return nb.value


def vsa_block_sparse_attn_fwd(q, k, v, row_ptr, col_idx, block_q, block_k, n_slabs=1, scale=None,
                              out=None, lse=None, want_lse=True, workspace=None, grouped=True, frame_tokens=None):
    """Exact softmax attention over the kept blocks -> (o, lse or None).

    With a workspace (allocated here unless given), small query blocks run grouped
    (several blocks per workgroup over the union of their kept blocks), and problems with
    too few rows to fill the chip split each row's key stream over several workgroups and
    merge the parts.  grouped=False runs without a workspace: neither grouped nor split
    (same results; bit for bit for grouped blocks of 65 to 128 rows, to rounding
    otherwise)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("row_ptr", row_ptr), ("col_idx", col_idx)):
        _require(t, name, q.device)
    B, nq, Hh, D = q.shape
    nk = k.shape[1]
    if k.shape != (B, nk, Hh, D) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v shapes / dtypes do not match")
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise ValueError("row_ptr and col_idx must be int32")
    if row_ptr.numel() != n_slabs * -(-nq // block_q) + 1:
        raise ValueError("row_ptr length does not match n_slabs * n_qblocks + 1")
    scale = D ** -0.5 if scale is None else scale
    out = torch.empty_like(q) if out is None else out
    _require(out, "out", q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hh, nq), dtype=torch.float32, device=q.device)
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _DTYPE[q.dtype], B, Hh, D, nq, nk, block_q, block_k)
    tail = (_ptr(row_ptr), _ptr(col_idx), n_slabs, float(scale))
    if frame_tokens is None:
        name, fn, args = "vsa_block_sparse_attn_fwd", lib().vsa_block_sparse_attn_fwd, head + tail
    else:
        name, fn, args = "vsa_radial_attn_fwd", lib().vsa_radial_attn_fwd, head + (int(frame_tokens),) + tail
    nb = ctypes.c_size_t(0)
    if grouped:
        if workspace is None:
            _check(fn(*args, None, ctypes.byref(nb), _stream(q)), name)
            if nb.value:
                workspace = torch.empty(nb.value, dtype=torch.uint8, device=q.device)
        if workspace is not None:
            _require(workspace, "workspace", q.device)
            nb = ctypes.c_size_t(workspace.numel())
    else:
        workspace = None
    _check(fn(*args, _ptr(workspace) if workspace is not None else None,
              ctypes.byref(nb) if workspace is not None else None, _stream(q)), name)
    return out, lse


def vsa_tiled_attn_fwd(q, k, v, grid, tile, row_ptr, col_idx, n_slabs=1, scale=None, out=None, lse=None,
                       want_lse=True, workspace=None, grouped=True):
    """Attention on raster-order tokens of a T x H x W grid whose tt x th x tw tiles (in
    tile-major order) are the blocks -> (o, lse or None), both in raster order.  Equals
    tile reorder -> vsa_block_sparse_attn_fwd -> inverse reorder, with the permutation
    applied to the row addresses inside the kernel instead of to the tensors."""
    for name, t in (("q", q), ("k", k), ("v", v), ("row_ptr", row_ptr), ("col_idx", col_idx)):
        _require(t, name, q.device)
    (T, H, W), (tt, th, tw) = grid, tile
    B, n, Hh, D = q.shape
    if n != T * H * W or k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be [batch, T*H*W, heads, head_dim] of one dtype")
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise ValueError("row_ptr and col_idx must be int32")
    n_tiles = (T // tt) * (H // th) * (W // tw)
    if row_ptr.numel() != n_slabs * n_tiles + 1:
        raise ValueError("row_ptr length does not match n_slabs * n_tiles + 1")
    scale = D ** -0.5 if scale is None else scale
    out = torch.empty_like(q) if out is None else out
    _require(out, "out", q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hh, n), dtype=torch.float32, device=q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _DTYPE[q.dtype], B, Hh, D, T, H, W, tt, th, tw,
            _ptr(row_ptr), _ptr(col_idx), n_slabs, float(scale))
    nb = ctypes.c_size_t(0)
    if grouped:
        if workspace is None:
            _check(lib().vsa_tiled_attn_fwd(*args, None, ctypes.byref(nb), _stream(q)), "vsa_tiled_attn_fwd")
            if nb.value:
                workspace = torch.empty(nb.value, dtype=torch.uint8, device=q.device)
        if workspace is not None:
            _require(workspace, "workspace", q.device)
            nb = ctypes.c_size_t(workspace.numel())
    else:
        workspace = None
    _check(lib().vsa_tiled_attn_fwd(*args, _ptr(workspace) if workspace is not None else None,
                                    ctypes.byref(nb) if workspace is not None else None, _stream(q)),
           "vsa_tiled_attn_fwd")
    return out, lse


def tiled_attn_workspace_bytes(q, grid, tile, row_ptr, col_idx, n_slabs=1):
    """Workspace bytes vsa_tiled_attn_fwd uses to group small tiles (0: none)."""
    (T, H, W), (tt, th, tw) = grid, tile
    B, n, Hh, D = q.shape
    nb = ctypes.c_size_t(0)
    _check(lib().vsa_tiled_attn_fwd(_ptr(q), _ptr(q), _ptr(q), _ptr(q), None, _DTYPE[q.dtype], B, Hh, D, T, H, W,
                                    tt, th, tw, _ptr(row_ptr), _ptr(col_idx), n_slabs, D ** -0.5, None,
                                    ctypes.byref(nb), _stream(q)), "vsa_tiled_attn_fwd")
    return nb.value


def attn_fwd_workspace_bytes(q, k, row_ptr, col_idx, block_q, block_k, n_slabs=1):
    """Workspace bytes the forward uses to group small query blocks (0: none)."""
    B, nq, Hh, D = q.shape
    nb = ctypes.c_size_t(0)
    _check(lib().vsa_block_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(k), _ptr(q), None, _DTYPE[q.dtype], B, Hh, D, nq,
                                           k.shape[1], block_q, block_k, _ptr(row_ptr), _ptr(col_idx), n_slabs,
                                           D ** -0.5, None, ctypes.byref(nb), _stream(q)), "vsa_block_sparse_attn_fwd")
    return nb.value


def all_ones_mask(n_qblocks, n_kblocks, device):
    """All-ones CSR (dense attention) built on the device with torch fills."""
    row_ptr = torch.arange(0, (n_qblocks + 1) * n_kblocks, n_kblocks, dtype=torch.int32, device=device)
    col_idx = torch.arange(n_kblocks, dtype=torch.int32, device=device).repeat(n_qblocks)
    return row_ptr, col_idx


def ar_forced_ranges(frame_tokens, n_frames, anchor_frames, recent_frames, block):
    """Key-block ranges [lo, hi) of the anchor frames and the most recent frames of a
    KV cache of n_frames frames (raster, `block`-token blocks)."""
    nbk = -(-(frame_tokens * n_frames) // block)
    return [(0, -(-(anchor_frames * frame_tokens) // block)),
            (((n_frames - recent_frames) * frame_tokens) // block, nbk)]

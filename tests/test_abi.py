"""C-ABI contract tests that need no GPU: the library loads, exports every call
the header declares, and rejects bad arguments on the host before any launch.

Every call below either fails validation or is a workspace-size query, so no
kernel is ever launched and the (fake, non-null) pointers are never touched."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_masks_amd as vsa
from block_sparse_attention_masks_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)      # 16-byte aligned, never dereferenced
ODD = ctypes.c_void_p(0x1008)       # misaligned
NULL = ctypes.c_void_p(0)

OK, E_NULL, E_SHAPE, E_DTYPE, E_PARAM, E_CAP, E_UNSUP = 0, -1, -2, -3, -4, -5, -6


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libvsa.so is not built (run __graft_entry__.build())")
    return vsa.lib()


def test_exports_match_header(L):
    with open(os.path.join(ROOT, "include", "vsa.h")) as f:
        header = f.read()
    declared = set(re.findall(r"^(?:vsa_status|const char\*)\s+(vsa_\w+)\(", header, re.M))
    assert declared == set(vsa.EXPORTS)
    for name in declared:
        assert hasattr(L, name)


def test_status_strings(L):
    for code in range(-7, 1):
        s = vsa.status_string(code)
        assert s.startswith("VSA_")
    assert "unknown" in vsa.status_string(-99)


def reorder(L, src=FAKE, dst=FAKE, batch=1, grid=(4, 8, 8), tile=(2, 4, 4), row_bytes=256, inverse=0):
    return L.vsa_tile_reorder(src, dst, batch, *grid, *tile, row_bytes, inverse, NULL)


def test_reorder_validation(L):
    assert reorder(L, src=NULL) == E_NULL
    assert reorder(L, dst=NULL) == E_NULL
    assert reorder(L, batch=0) == E_SHAPE
    assert reorder(L, grid=(5, 8, 8)) == E_SHAPE
    assert reorder(L, tile=(2, 0, 4)) == E_SHAPE
    assert reorder(L, inverse=2) == E_PARAM
    assert reorder(L, row_bytes=24) == E_UNSUP
    assert reorder(L, src=ODD) == E_UNSUP
    assert reorder(L, grid=(2048, 2048, 1024), tile=(1, 1, 1)) == E_SHAPE


def sta(L, grid=(8, 16, 16), tile=(4, 4, 4), window=(1, 3, 3), rp=FAKE, ci=FAKE, cap=10 ** 6):
    return L.vsa_mask_sta(*grid, *tile, *window, rp, ci, cap, NULL)


def test_sta_validation(L):
    assert sta(L, rp=NULL) == E_NULL
    assert sta(L, ci=NULL) == E_NULL
    assert sta(L, grid=(8, 16, 15)) == E_SHAPE
    assert sta(L, window=(2, 3, 3)) == E_PARAM
    assert sta(L, window=(1, 3, 0)) == E_PARAM
    assert sta(L, cap=32 * 9 - 1) == E_CAP          # bound = 32 tiles * 1*3*3


def radial(L, T=5, S=64, block=16, rp=FAKE, ci=FAKE, cap=10 ** 6):
    return L.vsa_mask_radial(T, S, block, rp, ci, cap, NULL)


def test_radial_validation(L):
    assert radial(L, rp=NULL) == E_NULL
    assert radial(L, T=0) == E_SHAPE
    assert radial(L, block=-1) == E_SHAPE
    assert radial(L, cap=20 * 20 - 1) == E_CAP
    assert radial(L, T=125, S=3600, block=1) == E_SHAPE   # nb^2 overflows int32


def nabla(L, q=FAKE, k=FAKE, dtype=1, B=1, H=2, D=128, nq=1000, nk=900, bq=64, bk=64, scale=0.1,
          thr=0.8, topk=0, forced=(), rp=FAKE, ci=FAKE, cap=10 ** 8, ws=FAKE, nbytes=None):
    sel, keep = _lib._select(thr, topk, forced)
    nb = ctypes.c_size_t(10 ** 12 if nbytes is None else nbytes)
    st = L.vsa_mask_nabla(q, k, dtype, B, H, D, nq, nk, bq, bk, scale, ctypes.byref(sel), rp, ci, cap,
                          ws, ctypes.byref(nb), NULL)
    return st, nb.value


def test_nabla_validation(L):
    assert nabla(L, q=NULL)[0] == E_NULL
    assert nabla(L, dtype=2)[0] == E_DTYPE
    assert nabla(L, D=96)[0] == E_UNSUP
    assert nabla(L, nq=0)[0] == E_SHAPE
    assert nabla(L, thr=0.0)[0] == E_PARAM
    assert nabla(L, thr=1.5)[0] == E_PARAM
    assert nabla(L, topk=-1)[0] == E_PARAM
    assert nabla(L, topk=4, forced=[(0, 3), (2, 5)])[0] == E_PARAM        # overlapping
    assert nabla(L, topk=4, forced=[(0, 30)])[0] == E_PARAM               # past n_kblocks (15)
    assert nabla(L, nk=64 * 5000)[0] == E_UNSUP
    assert nabla(L, nbytes=0)[0] == E_CAP
    assert nabla(L, cap=2 * 16 * 15 - 1)[0] == E_CAP
    assert nabla(L, q=ODD)[0] == E_UNSUP


def test_nabla_workspace_query(L):
    st, need = nabla(L, ws=NULL, nbytes=0)
    assert st == OK
    # pooled Q (2 heads x 16 blocks x 128 fp64), pooled K (2 x 15 x 128), map
    # (2 x 16 x 15 fp64), bitmap (32 rows x 1 word), each 256-byte aligned
    expect = sum(-(-x // 256) * 256 for x in (2 * 16 * 128 * 8, 2 * 15 * 128 * 8, 2 * 16 * 15 * 8, 32 * 4))
    assert need == expect


def attn(L, q=FAKE, k=FAKE, v=FAKE, o=FAKE, dtype=1, B=1, H=2, D=128, nq=100, nk=100, bq=64, bk=64,
         rp=FAKE, ci=FAKE, slabs=1, scale=0.1, ws=FAKE, query=False):
    nb = ctypes.c_size_t(123)
    st = L.vsa_block_sparse_attn_fwd(q, k, v, o, NULL, dtype, B, H, D, nq, nk, bq, bk, rp, ci, slabs,
                                     scale, NULL if query else ws, ctypes.byref(nb) if query else None, NULL)
    return st, nb.value


def test_attn_validation(L):
    assert attn(L, v=NULL)[0] == E_NULL
    assert attn(L, rp=NULL)[0] == E_NULL
    assert attn(L, dtype=7)[0] == E_DTYPE
    assert attn(L, D=32)[0] == E_UNSUP
    assert attn(L, nk=-1)[0] == E_SHAPE
    assert attn(L, nk=2 ** 31 - 64)[0] == E_SHAPE       # token counts stay below 2^31 - 64
    assert attn(L, nq=2 ** 31 - 64, bq=2 ** 20)[0] == E_SHAPE
    assert attn(L, bq=0)[0] == E_SHAPE
    assert attn(L, slabs=3)[0] == E_PARAM
    assert attn(L, scale=float("nan"))[0] == E_PARAM
    assert attn(L, scale=-0.1)[0] == E_PARAM
    assert attn(L, o=ODD)[0] == E_UNSUP
    # the size query reports the packed V^T (2 heads x 2 tiles of 64 keys x 128 x 2 bytes) ...
    assert attn(L, query=True) == (OK, 65536)
    # ... which fewer queries than keys, or key blocks that are not a multiple of 64, do not use
    assert attn(L, nq=99, query=True) == (OK, 0)
    assert attn(L, bk=96, query=True) == (OK, 0)
    # ... or whose packing grid (one workgroup per batch entry x 64-key tile) would pass 2^31 - 1
    assert attn(L, B=128, H=1, nq=2 ** 30, nk=2 ** 30, bq=2 ** 20, bk=2 ** 20, query=True) == (OK, 0)
    assert attn(L, B=127, H=1, nq=2 ** 30, nk=2 ** 30, bq=2 ** 20, bk=2 ** 20, query=True) == \
        (OK, 2 * 127 * 2 ** 24 * 64 * 128)
    # bf16 token rows of 2^24 bytes or more: the kernels' 24-bit row offsets would wrap
    assert attn(L, H=65536, D=128)[0] == E_UNSUP
    assert attn(L, H=65536, D=128, query=True)[0] == E_UNSUP
    assert attn(L, H=65535, D=128, query=True)[0] == OK
    assert attn(L, H=65536, D=128, dtype=0, query=True)[0] == OK      # fp32 path: no such limit


def test_static_attn_validation(L):
    """The allocation-free forward validates like the forward and refuses a problem whose
    workspace would exceed its 64 MiB array before it touches the device."""
    def st(q=FAKE, H=2, n=100, b=64, slabs=1, scale=0.1, dtype=1):
        return L.vsa_block_sparse_attn_fwd_static(q, FAKE, FAKE, FAKE, NULL, dtype, 1, H, 128, n, n, b, b, FAKE, FAKE,
                                                  slabs, scale, NULL)
    assert st(q=NULL) == E_NULL
    assert st(dtype=4) == E_DTYPE
    assert st(slabs=3) == E_PARAM
    assert st(scale=0.0) == E_PARAM
    assert st(q=ODD) == E_UNSUP
    # 256 heads x 30,000 tokens in 64-token blocks, per-head masks: 75.9 MB of union lists
    assert st(H=256, n=30000, slabs=256) == E_CAP


def tiled(L, q=FAKE, dtype=1, B=1, H=2, D=128, grid=(12, 16, 16), tile=(6, 8, 8), rp=FAKE, ci=FAKE, slabs=1,
          scale=0.1, query=False):
    nb = ctypes.c_size_t(123)
    st = L.vsa_tiled_attn_fwd(q, FAKE, FAKE, FAKE, NULL, dtype, B, H, D, *grid, *tile, rp, ci, slabs, scale,
                              NULL if query else FAKE, ctypes.byref(nb) if query else None, NULL)
    return st, nb.value


def test_tiled_attn_validation(L):
    assert tiled(L, q=NULL)[0] == E_NULL
    assert tiled(L, ci=NULL)[0] == E_NULL
    assert tiled(L, grid=(12, 16, 15))[0] == E_SHAPE       # W not divisible by tw
    assert tiled(L, grid=(0, 16, 16))[0] == E_SHAPE
    assert tiled(L, grid=(2048, 1024, 1024), tile=(1, 8, 8))[0] == E_SHAPE   # 2^31 tokens
    assert tiled(L, dtype=5)[0] == E_DTYPE
    assert tiled(L, D=96)[0] == E_UNSUP
    assert tiled(L, slabs=3)[0] == E_PARAM
    assert tiled(L, scale=0.0)[0] == E_PARAM
    assert tiled(L, q=ODD)[0] == E_UNSUP
    # tile planes that do not nest with the 64-token copy tile
    assert tiled(L, grid=(9, 9, 9), tile=(3, 3, 3))[0] == E_UNSUP
    assert tiled(L, grid=(2, 4, 192), tile=(1, 2, 96))[0] == E_UNSUP
    # supported planes: 64 | th*tw with tw | 64, tw a multiple of 64, th*tw | 64
    for grid, tile in (((12, 16, 16), (6, 8, 8)), ((2, 24, 32), (1, 12, 16)), ((2, 4, 256), (1, 1, 128)),
                       ((8, 8, 8), (4, 4, 4)), ((4, 4, 4), (1, 1, 1))):
        assert tiled(L, grid=grid, tile=tile, query=True)[0] == OK
    # tiles of more than 4096 tokens
    assert tiled(L, grid=(16, 16, 32), tile=(16, 16, 32), query=True)[0] == E_UNSUP
    assert tiled(L, grid=(16, 16, 16), tile=(16, 16, 16), query=True)[0] == OK
    # bf16 copy-tile lane offsets must fit 32-bit bytes and 24-bit rows: 1x1x1 tiles put a
    # copy tile's 64 rows 64 planes apart (63 * 1024 * 1024 rows of 128 bytes > 4 GiB)
    assert tiled(L, grid=(64, 1024, 1024), tile=(1, 1, 1), H=1, D=64)[0] == E_UNSUP
    assert tiled(L, grid=(64, 256, 256), tile=(1, 1, 1), H=1, D=64, query=True)[0] == OK
    assert tiled(L, grid=(64, 1024, 1024), tile=(1, 1, 1), H=1, D=64, dtype=0, query=True)[0] == OK  # fp32 path
    # workspace: none for 384-token tiles, the union lists for 64-token tiles (grouped)
    # the packed V^T: 12 x 16 x 16 tokens = 48 tiles of 64 keys, 2 heads, 128 x 2 bytes each
    assert tiled(L, query=True) == (OK, 48 * 2 * 64 * 128 * 2)
    assert tiled(L, grid=(12, 64, 64), tile=(1, 8, 8), query=True)[1] > 0


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 64, 2, 8)
    with pytest.raises(ValueError):
        vsa.vsa_tile_reorder(x, (4, 4, 4), (2, 2, 2))


def sta_heads(L, grid=(8, 16, 16), tile=(4, 4, 4), windows=((1, 3, 3), (3, 3, 1)), batch=2,
              rp=FAKE, ci=FAKE, cap=10 ** 6, null_windows=False):
    flat = [x for w in windows for x in w]
    arr = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    wptr = NULL if null_windows else ctypes.cast(arr, ctypes.c_void_p)
    return L.vsa_mask_sta_heads(*grid, *tile, wptr, len(windows), batch, rp, ci, cap, NULL)


def test_sta_heads_validation(L):
    assert sta_heads(L, null_windows=True) == E_NULL
    assert sta_heads(L, rp=NULL) == E_NULL
    assert sta_heads(L, grid=(8, 16, 15)) == E_SHAPE
    assert sta_heads(L, batch=0) == E_SHAPE
    assert sta_heads(L, windows=((1, 3, 3), (2, 3, 3))) == E_PARAM
    assert sta_heads(L, windows=((1, 3, 3), (1, -1, 3))) == E_PARAM
    assert sta_heads(L, windows=((1, 1, 1),) * 257) == E_UNSUP
    # bound = batch * (32 tiles * 1*3*3 + 32 tiles * 2*3*1): windows clipped to the 2x4x4 grid
    assert sta_heads(L, cap=2 * (32 * 9 + 32 * 6) - 1) == E_CAP


def union(L, nq=10, nk=7, rpa=FAKE, cia=FAKE, sa=1, rpb=FAKE, cib=FAKE, sb=4, rp=FAKE, ci=FAKE, cap=10 ** 6):
    return L.vsa_mask_union(nq, nk, rpa, cia, sa, rpb, cib, sb, rp, ci, cap, NULL)


def test_union_validation(L):
    assert union(L, cia=NULL) == E_NULL
    assert union(L, ci=NULL) == E_NULL
    assert union(L, nq=0) == E_SHAPE
    assert union(L, sa=0) == E_SHAPE
    assert union(L, sa=2, sb=4) == E_PARAM
    assert union(L, cap=4 * 10 * 7 - 1) == E_CAP
    assert union(L, nq=2 ** 20, nk=2 ** 12, sb=1) == E_SHAPE


def sics(L, x=FAKE, dtype=1, B=1, H=2, D=128, n=1000, block=64, out=FAKE):
    return L.vsa_block_sics(x, dtype, B, H, D, n, block, out, NULL)


def test_mean_pool_validation(L):
    def pool(x=FAKE, dtype=1, B=1, H=2, D=128, n=100, block=64, out=FAKE):
        return L.vsa_block_mean_pool(x, dtype, B, H, D, n, block, out, NULL)
    assert pool(x=NULL) == E_NULL
    assert pool(out=NULL) == E_NULL
    assert pool(dtype=5) == E_DTYPE
    assert pool(n=0) == E_SHAPE
    assert pool(block=-1) == E_SHAPE
    assert pool(B=65536) == E_SHAPE
    assert pool(D=96) == E_UNSUP
    assert pool(x=ODD) == E_UNSUP
    assert pool(out=ctypes.c_void_p(0x1004)) == E_UNSUP


def test_sics_validation(L):
    assert sics(L, x=NULL) == E_NULL
    assert sics(L, out=NULL) == E_NULL
    assert sics(L, dtype=5) == E_DTYPE
    assert sics(L, D=96) == E_UNSUP
    assert sics(L, n=0) == E_SHAPE
    assert sics(L, block=0) == E_SHAPE
    assert sics(L, x=ODD) == E_UNSUP


def test_kv_validation(L):
    assert L.vsa_kv_plan(NULL, FAKE, 1, 4, 1000, 64, FAKE, FAKE, NULL) == E_NULL
    assert L.vsa_kv_plan(FAKE, FAKE, 0, 4, 1000, 64, FAKE, FAKE, NULL) == E_SHAPE
    assert L.vsa_kv_plan(FAKE, FAKE, 1, 4, 1000, 0, FAKE, FAKE, NULL) == E_SHAPE
    g = lambda **kw: L.vsa_kv_gather(kw.get("x", FAKE), kw.get("dtype", 1), 1, 2, kw.get("D", 128), 1000, 64,
                                     FAKE, kw.get("slabs", 2), kw.get("out", FAKE), kw.get("n_out", 500), NULL)
    assert g(x=NULL) == E_NULL
    assert g(dtype=3) == E_DTYPE
    assert g(D=80) == E_UNSUP
    assert g(slabs=3) == E_PARAM
    assert g(n_out=0) == E_SHAPE
    assert g(out=ODD) == E_UNSUP
    assert L.vsa_mask_remap(FAKE, FAKE, 1, 4, NULL, 16, FAKE, NULL) == E_NULL
    assert L.vsa_mask_remap(FAKE, FAKE, 1, 0, FAKE, 16, FAKE, NULL) == E_SHAPE


def bwd(L, q=FAKE, dtype=1, H=2, D=128, slabs=1, scale=0.1, ws=FAKE, nbytes=10 ** 9, dq=FAKE, query=False):
    nb = ctypes.c_size_t(nbytes)
    st = L.vsa_block_sparse_attn_bwd(q, FAKE, FAKE, FAKE, FAKE, FAKE, dq, FAKE, FAKE, dtype, 1, H, D, 100, 90,
                                     64, 64, FAKE, FAKE, slabs, scale, NULL if query else ws, ctypes.byref(nb), NULL)
    return st, nb.value


def test_bwd_validation(L):
    assert bwd(L, q=NULL)[0] == E_NULL
    assert bwd(L, dtype=9)[0] == E_DTYPE
    assert bwd(L, D=48)[0] == E_UNSUP
    assert bwd(L, slabs=3)[0] == E_PARAM
    assert bwd(L, scale=0.0)[0] == E_PARAM
    st, need = bwd(L, query=True)
    assert st == OK
    # D per query, CSC counters and pointers, query-block indices (dense bound), 256-byte aligned
    expect = sum(-(-x // 256) * 256 for x in (4 * 2 * 100, 4 * 2, 4 * 3, 4 * 2 * 2))
    assert need == expect
    assert bwd(L, nbytes=need - 1)[0] == E_CAP
    assert bwd(L, dq=NULL)[0] == E_NULL
    assert bwd(L, dq=ODD)[0] == E_UNSUP
    assert bwd(L, H=65536, query=True)[0] == E_UNSUP                 # bf16 rows of 2^24 bytes
    assert bwd(L, H=65535, query=True)[0] == OK


C_CALLER = r"""
#include "vsa.h"
#include <stdio.h>
/* a C caller: the header parses as C and the library links; no call here reaches a kernel */
int main(void) {
  printf("%s\n", vsa_status_string(VSA_ERR_SHAPE));
  if (vsa_mask_radial(0, 0, 0, 0, 0, 0, 0) != VSA_ERR_NULL) return 1;
  size_t need = 0;
  vsa_select sel = {0.9, 0, 0, 0};
  (void)sel;
  if (vsa_block_sparse_attn_fwd(0, 0, 0, 0, 0, VSA_BF16, 1, 1, 128, 1, 1, 64, 64, 0, 0, 1, 1.0f, 0, &need, 0) !=
      VSA_ERR_NULL)
    return 2;
  return 0;
}
"""


@pytest.mark.parametrize("compiler,std", [("gcc", "-std=c99"), ("g++", "-std=c++17")])
def test_header_compiles_and_links_from_c(L, tmp_path, compiler, std):
    """include/vsa.h as a C (and C++) caller sees it: it compiles warning-free, the program links
    against libvsa.so by the declared names, and the calls return the documented codes."""
    import shutil
    import subprocess
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not available")
    src = tmp_path / ("caller.c" if compiler == "gcc" else "caller.cpp")
    src.write_text(C_CALLER)
    exe = tmp_path / "caller"
    libdir = os.path.dirname(_lib.LIB_PATH)
    cmd = [compiler, std, "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", str(src), "-o", str(exe), "-L", libdir, f"-l:{os.path.basename(_lib.LIB_PATH)}",
           f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.strip() == _lib.status_string(E_SHAPE)

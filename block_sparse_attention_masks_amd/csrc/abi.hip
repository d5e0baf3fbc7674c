// C ABI of libvsa: argument validation on the host, then kernel launches on the
// caller's stream.  Nothing is launched unless every check passes.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "../../include/vsa.h"
#include "vsa_internal.h"

// Workspace of vsa_block_sparse_attn_fwd_static, for callers that cannot allocate: one
// array on every GPU the library runs on, held until the process ends.  Host code never
// uses the array's name as an address: static_scratch() resolves the device address.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

// The device address of `scratch` on the current device, resolved once per device with
// that device current (each GPU holds its own copy at its own address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

constexpr int64_t kI32Max = 2147483647;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

vsa_status from_hip(hipError_t e) { return e == hipSuccess ? VSA_OK : VSA_ERR_HIP; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The bf16 attention kernels address the rows of a 64-key tile as a 24-bit row index
// times a 24-bit row size: a token row (heads * head_dim bf16 values) must stay below
// 2^24 bytes.
bool bf16_rows_fit(int32_t heads, int32_t head_dim) { return (int64_t)heads * head_dim * 2 < (1 << 24); }

// Common checks of a token-tensor problem (dtype, head_dim, sizes).
vsa_status check_tokens(int32_t dtype, int64_t batch, int32_t heads, int32_t head_dim, int64_t nq,
                        int64_t nk, int32_t block_q, int32_t block_k) {
  if (dtype != VSA_F32 && dtype != VSA_BF16) return VSA_ERR_DTYPE;
  if (batch <= 0 || heads <= 0 || head_dim <= 0 || nq <= 0 || nk <= 0 || block_q <= 0 ||
      block_k <= 0)
    return VSA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return VSA_ERR_UNSUPPORTED;
  if (nq > kI32Max - 64 || nk > kI32Max - 64) return VSA_ERR_SHAPE;  // 64-key tiles step in 31 bits
  if (batch * heads * ceil_div(nq, block_q) > kI32Max) return VSA_ERR_SHAPE;
  return VSA_OK;
}

}  // namespace

extern "C" {

const char* vsa_status_string(vsa_status s) {
  switch (s) {
    case VSA_OK: return "VSA_OK";
    case VSA_ERR_NULL: return "VSA_ERR_NULL: a required pointer is NULL";
    case VSA_ERR_SHAPE: return "VSA_ERR_SHAPE: invalid or inconsistent sizes";
    case VSA_ERR_DTYPE: return "VSA_ERR_DTYPE: dtype must be VSA_F32 or VSA_BF16";
    case VSA_ERR_PARAM: return "VSA_ERR_PARAM: invalid mask or selection parameter";
    case VSA_ERR_CAPACITY: return "VSA_ERR_CAPACITY: output capacity or workspace too small";
    case VSA_ERR_UNSUPPORTED: return "VSA_ERR_UNSUPPORTED: head_dim, alignment or size not supported";
    case VSA_ERR_HIP: return "VSA_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown vsa_status";
  }
}

vsa_status vsa_tile_reorder(const void* src, void* dst, int64_t batch, int32_t T, int32_t H,
                            int32_t W, int32_t tt, int32_t th, int32_t tw, int64_t row_bytes,
                            int32_t inverse, hipStream_t stream) {
  if (!src || !dst) return VSA_ERR_NULL;
  if (batch <= 0 || T <= 0 || H <= 0 || W <= 0 || tt <= 0 || th <= 0 || tw <= 0 || row_bytes <= 0)
    return VSA_ERR_SHAPE;
  if (T % tt || H % th || W % tw) return VSA_ERR_SHAPE;
  if ((int64_t)T * H * W > kI32Max) return VSA_ERR_SHAPE;
  if (inverse != 0 && inverse != 1) return VSA_ERR_PARAM;
  if (row_bytes % 16 || !aligned16(src) || !aligned16(dst)) return VSA_ERR_UNSUPPORTED;
  if (row_bytes / 16 > kI32Max) return VSA_ERR_UNSUPPORTED;
  return from_hip(vsa::launch_tile_reorder(src, dst, batch, T, H, W, tt, th, tw, row_bytes, inverse,
                                           stream));
}

vsa_status vsa_mask_sta(int32_t T, int32_t H, int32_t W, int32_t tt, int32_t th, int32_t tw,
                        int32_t wt, int32_t wh, int32_t ww, int32_t* row_ptr, int32_t* col_idx,
                        int64_t col_capacity, hipStream_t stream) {
  if (!row_ptr || !col_idx) return VSA_ERR_NULL;
  if (T <= 0 || H <= 0 || W <= 0 || tt <= 0 || th <= 0 || tw <= 0) return VSA_ERR_SHAPE;
  if (T % tt || H % th || W % tw) return VSA_ERR_SHAPE;
  if (wt <= 0 || wh <= 0 || ww <= 0 || wt % 2 == 0 || wh % 2 == 0 || ww % 2 == 0)
    return VSA_ERR_PARAM;
  const int64_t NT = T / tt, NH = H / th, NW = W / tw, n = NT * NH * NW;
  const int64_t bound = n * std::min<int64_t>(wt, NT) * std::min<int64_t>(wh, NH) *
                        std::min<int64_t>(ww, NW);
  if (n > kI32Max || bound > kI32Max) return VSA_ERR_SHAPE;
  if (col_capacity < bound) return VSA_ERR_CAPACITY;
  return from_hip(vsa::launch_mask_sta((int)NT, (int)NH, (int)NW, wt / 2, wh / 2, ww / 2, row_ptr,
                                       col_idx, stream));
}

vsa_status vsa_mask_radial(int32_t T, int32_t S, int32_t block, int32_t* row_ptr,
                           int32_t* col_idx, int64_t col_capacity, hipStream_t stream) {
  if (!row_ptr || !col_idx) return VSA_ERR_NULL;
  if (T <= 0 || S <= 0 || block <= 0) return VSA_ERR_SHAPE;
  const int64_t N = (int64_t)T * S;
  if (N > kI32Max - block) return VSA_ERR_SHAPE;
  const int64_t nb = ceil_div(N, block);
  if (nb * nb > kI32Max) return VSA_ERR_SHAPE;
  if (col_capacity < nb * nb) return VSA_ERR_CAPACITY;
  return from_hip(vsa::launch_mask_radial(T, S, block, row_ptr, col_idx, stream));
}

vsa_status vsa_mask_sta_heads(int32_t T, int32_t H, int32_t W, int32_t tt, int32_t th, int32_t tw,
                              const int32_t* windows, int32_t heads, int64_t batch, int32_t* row_ptr,
                              int32_t* col_idx, int64_t col_capacity, hipStream_t stream) {
  if (!windows || !row_ptr || !col_idx) return VSA_ERR_NULL;
  if (T <= 0 || H <= 0 || W <= 0 || tt <= 0 || th <= 0 || tw <= 0 || heads <= 0 || batch <= 0)
    return VSA_ERR_SHAPE;
  if (T % tt || H % th || W % tw) return VSA_ERR_SHAPE;
  if (heads > vsa::kMaxStaHeads) return VSA_ERR_UNSUPPORTED;
  const int64_t NT = T / tt, NH = H / th, NW = W / tw, n = NT * NH * NW;
  if (n > kI32Max || batch * heads * n > kI32Max) return VSA_ERR_SHAPE;
  vsa::StaHeads p{};
  p.NT = (int)NT, p.NH = (int)NH, p.NW = (int)NW, p.heads = heads;
  const int64_t axis[3] = {NT, NH, NW};
  int64_t per_batch = 0;
  for (int h = 0; h < heads; ++h) {
    int64_t vol = n;
    for (int d = 0; d < 3; ++d) {
      const int32_t w = windows[3 * h + d];
      if (w <= 0 || w % 2 == 0) return VSA_ERR_PARAM;
      // a half-width past the axis length keeps the whole axis, as the clipped window does
      p.half[h][d] = (int16_t)std::min<int64_t>(w / 2, axis[d]);
      vol *= std::min<int64_t>(w, axis[d]);
    }
    per_batch += vol;
  }
  const int64_t bound = batch * per_batch;
  if (bound > kI32Max) return VSA_ERR_SHAPE;
  if (col_capacity < bound) return VSA_ERR_CAPACITY;
  return from_hip(vsa::launch_mask_sta_heads(p, batch * heads * n, row_ptr, col_idx, stream));
}

vsa_status vsa_mask_union(int64_t n_qblocks, int32_t n_kblocks, const int32_t* row_ptr_a,
                          const int32_t* col_idx_a, int64_t slabs_a, const int32_t* row_ptr_b,
                          const int32_t* col_idx_b, int64_t slabs_b, int32_t* row_ptr,
                          int32_t* col_idx, int64_t col_capacity, hipStream_t stream) {
  if (!row_ptr_a || !col_idx_a || !row_ptr_b || !col_idx_b || !row_ptr || !col_idx) return VSA_ERR_NULL;
  if (n_qblocks <= 0 || n_kblocks <= 0 || slabs_a <= 0 || slabs_b <= 0) return VSA_ERR_SHAPE;
  const int64_t slabs = std::max(slabs_a, slabs_b);
  if ((slabs_a != 1 && slabs_a != slabs) || (slabs_b != 1 && slabs_b != slabs)) return VSA_ERR_PARAM;
  if (slabs > kI32Max / n_qblocks) return VSA_ERR_SHAPE;
  const int64_t rows = slabs * n_qblocks;
  if (rows * n_kblocks > kI32Max) return VSA_ERR_SHAPE;
  if (col_capacity < rows * n_kblocks) return VSA_ERR_CAPACITY;
  const vsa::UnionArgs u{row_ptr_a, col_idx_a, row_ptr_b, col_idx_b, slabs_a, slabs_b, n_qblocks};
  return from_hip(vsa::launch_mask_union(u, rows, row_ptr, col_idx, stream));
}

vsa_status vsa_block_sics(const void* x, int32_t dtype, int64_t batch, int32_t heads, int32_t head_dim,
                          int64_t n, int32_t block, double* scores, hipStream_t stream) {
  if (!x || !scores) return VSA_ERR_NULL;
  const vsa_status st = check_tokens(dtype, batch, heads, head_dim, n, n, block, block);
  if (st != VSA_OK) return st;
  if (!aligned16(x)) return VSA_ERR_UNSUPPORTED;
  if (ceil_div(n, block) * ceil_div((int64_t)heads * head_dim, 512) > kI32Max || batch > 65535)
    return VSA_ERR_SHAPE;
  return from_hip(vsa::launch_block_sics(x, dtype == VSA_BF16, batch, heads, head_dim, n, block, scores,
                                         stream));
}

vsa_status vsa_kv_plan(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_slabs, int64_t n_qblocks,
                       int64_t nk, int32_t block_k, int32_t* slot, int32_t* info, hipStream_t stream) {
  if (!row_ptr || !col_idx || !slot || !info) return VSA_ERR_NULL;
  if (n_slabs <= 0 || n_qblocks <= 0 || nk <= 0 || block_k <= 0) return VSA_ERR_SHAPE;
  const int64_t nbk = ceil_div(nk, block_k);
  if (nbk > kI32Max || n_slabs > kI32Max || n_slabs * n_qblocks > kI32Max) return VSA_ERR_SHAPE;
  const int tail = nk % block_k ? (int)nbk - 1 : -1;
  return from_hip(vsa::launch_kv_plan(row_ptr, col_idx, n_slabs, n_qblocks, (int)nbk, tail, slot, info, stream));
}

vsa_status vsa_kv_gather(const void* x, int32_t dtype, int64_t batch, int32_t heads, int32_t head_dim,
                         int64_t nk, int32_t block_k, const int32_t* slot, int64_t n_slabs, void* out,
                         int64_t n_out, hipStream_t stream) {
  if (!x || !slot || !out) return VSA_ERR_NULL;
  const vsa_status st = check_tokens(dtype, batch, heads, head_dim, nk, nk, block_k, block_k);
  if (st != VSA_OK) return st;
  if (n_out <= 0 || n_out > kI32Max || batch > 65535) return VSA_ERR_SHAPE;
  if (n_slabs != 1 && n_slabs != batch * heads) return VSA_ERR_PARAM;
  if (!aligned16(x) || !aligned16(out)) return VSA_ERR_UNSUPPORTED;
  const int64_t nbk = ceil_div(nk, block_k);
  if (nbk * ((block_k + 7) / 8) > kI32Max) return VSA_ERR_SHAPE;
  const int esz = dtype == VSA_BF16 ? 2 : 4;
  const int row_vec = heads * head_dim * esz / 16;
  return from_hip(vsa::launch_kv_gather(x, batch, nk, block_k, heads, row_vec, (int)nbk, slot, n_slabs, out,
                                        n_out, stream));
}

vsa_status vsa_mask_remap(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_slabs, int64_t n_qblocks,
                          const int32_t* slot, int32_t n_kblocks, int32_t* col_out, hipStream_t stream) {
  if (!row_ptr || !col_idx || !slot || !col_out) return VSA_ERR_NULL;
  if (n_slabs <= 0 || n_qblocks <= 0 || n_kblocks <= 0) return VSA_ERR_SHAPE;
  if (n_slabs * n_qblocks > kI32Max) return VSA_ERR_SHAPE;
  return from_hip(vsa::launch_mask_remap(row_ptr, col_idx, n_slabs * n_qblocks, n_qblocks, slot, n_kblocks,
                                         n_slabs, col_out, stream));
}

vsa_status vsa_block_mean_pool(const void* x, int32_t dtype, int64_t batch, int32_t heads, int32_t head_dim,
                               int64_t n, int32_t block, double* out, hipStream_t stream) {
  if (!x || !out) return VSA_ERR_NULL;
  const vsa_status st = check_tokens(dtype, batch, heads, head_dim, n, n, block, block);
  if (st != VSA_OK) return st;
  if (batch > 65535 || ceil_div(n, block) * ceil_div((int64_t)heads * head_dim, 512) > kI32Max)
    return VSA_ERR_SHAPE;
  if (!aligned16(x) || ((uintptr_t)out & 7u)) return VSA_ERR_UNSUPPORTED;
  return from_hip(vsa::launch_block_pool(x, dtype == VSA_BF16, batch, heads, head_dim, n, block, out, stream));
}

vsa_status vsa_mask_nabla(const void* q, const void* k, int32_t dtype, int64_t batch,
                          int32_t heads, int32_t head_dim, int64_t nq, int64_t nk,
                          int32_t block_q, int32_t block_k, double scale, const vsa_select* sel,
                          int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                          void* workspace, size_t* workspace_bytes, hipStream_t stream) {
  if (!q || !k || !sel || !row_ptr || !col_idx || !workspace_bytes) return VSA_ERR_NULL;
  vsa_status st = check_tokens(dtype, batch, heads, head_dim, nq, nk, block_q, block_k);
  if (st != VSA_OK) return st;
  const int64_t nbq = ceil_div(nq, block_q), nbk = ceil_div(nk, block_k);
  if (batch > 65535 || (nbq + nbk) * ceil_div((int64_t)heads * head_dim, 512) > kI32Max) return VSA_ERR_SHAPE;
  if (nbk > 4096) return VSA_ERR_UNSUPPORTED;
  if (!(scale == scale)) return VSA_ERR_PARAM;
  if (sel->topk < 0 || sel->n_forced < 0 || sel->n_forced > 16) return VSA_ERR_PARAM;
  if (sel->topk == 0 && !(sel->cdf_threshold > 0.0 && sel->cdf_threshold <= 1.0))
    return VSA_ERR_PARAM;
  if (sel->topk > 0 && sel->n_forced > 0) {
    if (!sel->forced) return VSA_ERR_NULL;
    for (int r = 0; r < sel->n_forced; ++r) {
      const int lo = sel->forced[2 * r], hi = sel->forced[2 * r + 1];
      if (lo < 0 || hi > nbk || lo > hi) return VSA_ERR_PARAM;
      for (int u = 0; u < r; ++u)  // ranges must be disjoint
        if (lo < sel->forced[2 * u + 1] && sel->forced[2 * u] < hi) return VSA_ERR_PARAM;
    }
  }
  const int64_t rows = batch * heads * nbq;
  if (rows * nbk > kI32Max) return VSA_ERR_SHAPE;
  const size_t need = vsa::nabla_workspace_bytes(batch, heads, head_dim, nq, nk, block_q, block_k);
  if (!workspace) {
    *workspace_bytes = need;
    return VSA_OK;
  }
  if (*workspace_bytes < need) return VSA_ERR_CAPACITY;
  if (col_capacity < rows * nbk) return VSA_ERR_CAPACITY;
  if (!aligned16(q) || !aligned16(k) || !aligned16(workspace)) return VSA_ERR_UNSUPPORTED;
  vsa::NablaArgs a{q, k, dtype, batch, heads, head_dim, nq, nk, block_q, block_k, scale,
                   sel->cdf_threshold, sel->topk, sel->n_forced, sel->forced, row_ptr, col_idx,
                   workspace};
  return from_hip(vsa::launch_mask_nabla(a, stream));
}

}  // extern "C"

namespace {

// The forward on untiled tokens, with query blocks grouped `group_stride` blocks apart.
vsa_status attn_fwd_untiled(const void* q, const void* k, const void* v, void* o, float* lse, int32_t dtype,
                            int64_t batch, int32_t heads, int32_t head_dim, int64_t nq, int64_t nk,
                            int32_t block_q, int32_t block_k, const int32_t* row_ptr, const int32_t* col_idx,
                            int32_t n_slabs, float scale, int group_stride, void* workspace,
                            size_t* workspace_bytes, hipStream_t stream, bool use_static = false) {
  if (!q || !k || !v || !o || !row_ptr || !col_idx) return VSA_ERR_NULL;
  vsa_status st = check_tokens(dtype, batch, heads, head_dim, nq, nk, block_q, block_k);
  if (st != VSA_OK) return st;
  if (n_slabs != 1 && (int64_t)n_slabs != batch * heads) return VSA_ERR_PARAM;
  if (!(scale > 0.0f) || scale == INFINITY) return VSA_ERR_PARAM;
  if (dtype == VSA_BF16 && !bf16_rows_fit(heads, head_dim)) return VSA_ERR_UNSUPPORTED;
  vsa::AttnArgs a{q, k, v, o, lse, dtype, batch, heads, head_dim, nq, nk, block_q, block_k,
                  row_ptr, col_idx, n_slabs, scale};
  a.group_stride = group_stride;
  const size_t want = dtype == VSA_BF16 ? vsa::attn_fwd_workspace(a) : 0;
  if (use_static) {  // the file-scope scratch array, never an allocation
    // the packed V^T is optional: it is used only when the scratch holds it too
    if (dtype == VSA_BF16 && vsa::attn_fwd_workspace_min(a) > kStaticScratchBytes) return VSA_ERR_CAPACITY;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return VSA_ERR_UNSUPPORTED;
    void* ws = nullptr;
    if (want > 0) {
      const hipError_t e = static_scratch(&ws);
      if (e != hipSuccess) return VSA_ERR_HIP;
    }
    return from_hip(vsa::launch_attn_fwd(a, ws, ws ? kStaticScratchBytes : 0, stream));
  }
  if (workspace_bytes && !workspace) {  // size query
    *workspace_bytes = want;
    return VSA_OK;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return VSA_ERR_UNSUPPORTED;
  if (workspace && ((uintptr_t)workspace & 255u)) return VSA_ERR_UNSUPPORTED;
  const size_t have = workspace && workspace_bytes ? *workspace_bytes : 0;
  return from_hip(vsa::launch_attn_fwd(a, workspace, have, stream));
}

}  // namespace

extern "C" {

vsa_status vsa_block_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int32_t dtype, int64_t batch, int32_t heads,
                                     int32_t head_dim, int64_t nq, int64_t nk, int32_t block_q,
                                     int32_t block_k, const int32_t* row_ptr,
                                     const int32_t* col_idx, int32_t n_slabs, float scale,
                                     void* workspace, size_t* workspace_bytes,
                                     hipStream_t stream) {
  return attn_fwd_untiled(q, k, v, o, lse, dtype, batch, heads, head_dim, nq, nk, block_q, block_k, row_ptr,
                          col_idx, n_slabs, scale, 1, workspace, workspace_bytes, stream);
}

vsa_status vsa_block_sparse_attn_fwd_static(const void* q, const void* k, const void* v, void* o, float* lse,
                                            int32_t dtype, int64_t batch, int32_t heads, int32_t head_dim,
                                            int64_t nq, int64_t nk, int32_t block_q, int32_t block_k,
                                            const int32_t* row_ptr, const int32_t* col_idx, int32_t n_slabs,
                                            float scale, hipStream_t stream) {
  return attn_fwd_untiled(q, k, v, o, lse, dtype, batch, heads, head_dim, nq, nk, block_q, block_k, row_ptr,
                          col_idx, n_slabs, scale, 1, nullptr, nullptr, stream, true);
}

vsa_status vsa_radial_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int32_t dtype,
                               int64_t batch, int32_t heads, int32_t head_dim, int64_t nq, int64_t nk,
                               int32_t block_q, int32_t block_k, int64_t frame_tokens, const int32_t* row_ptr,
                               const int32_t* col_idx, int32_t n_slabs, float scale, void* workspace,
                               size_t* workspace_bytes, hipStream_t stream) {
  if (frame_tokens <= 0 || block_q <= 0) return VSA_ERR_SHAPE;
  const int64_t stride = std::max<int64_t>(1, frame_tokens / block_q);
  if (stride > kI32Max / 16) return VSA_ERR_SHAPE;
  return attn_fwd_untiled(q, k, v, o, lse, dtype, batch, heads, head_dim, nq, nk, block_q, block_k, row_ptr,
                          col_idx, n_slabs, scale, (int)stride, workspace, workspace_bytes, stream);
}

vsa_status vsa_tiled_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                              int32_t dtype, int64_t batch, int32_t heads, int32_t head_dim,
                              int32_t T, int32_t H, int32_t W, int32_t tt, int32_t th, int32_t tw,
                              const int32_t* row_ptr, const int32_t* col_idx, int32_t n_slabs,
                              float scale, void* workspace, size_t* workspace_bytes,
                              hipStream_t stream) {
  if (!q || !k || !v || !o || !row_ptr || !col_idx) return VSA_ERR_NULL;
  if (T <= 0 || H <= 0 || W <= 0 || tt <= 0 || th <= 0 || tw <= 0) return VSA_ERR_SHAPE;
  if (T % tt || H % th || W % tw) return VSA_ERR_SHAPE;
  const int64_t n = (int64_t)T * H * W, block = (int64_t)tt * th * tw;
  if (n > kI32Max || block > kI32Max) return VSA_ERR_SHAPE;
  vsa_status st = check_tokens(dtype, batch, heads, head_dim, n, n, (int32_t)block, (int32_t)block);
  if (st != VSA_OK) return st;
  if (n_slabs != 1 && (int64_t)n_slabs != batch * heads) return VSA_ERR_PARAM;
  if (!(scale > 0.0f) || scale == INFINITY) return VSA_ERR_PARAM;
  if (vsa::tiling_mode(th, tw) == 0 || block > 64 * vsa::kTiledMaxCopyTiles) return VSA_ERR_UNSUPPORTED;
  // bf16: a copy tile's lane offsets (rows after its first token) are 24-bit rows and
  // 32-bit bytes
  const int64_t row_bytes = (int64_t)heads * head_dim * 2, span = vsa::tiling_lane_span(H, W, th, tw);
  if (dtype == VSA_BF16 && (span >= (1 << 24) || !bf16_rows_fit(heads, head_dim) || (span + 1) * row_bytes > (int64_t)UINT32_MAX))
    return VSA_ERR_UNSUPPORTED;
  vsa::AttnArgs a{q, k, v, o, lse, dtype, batch, heads, head_dim, n, n, (int)block, (int)block,
                  row_ptr, col_idx, n_slabs, scale};
  a.tiled = 1;
  a.H = H;
  a.W = W;
  a.tt = tt;
  a.th = th;
  a.tw = tw;
  const size_t want = dtype == VSA_BF16 ? vsa::attn_fwd_workspace(a) : 0;
  if (workspace_bytes && !workspace) {  // size query
    *workspace_bytes = want;
    return VSA_OK;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return VSA_ERR_UNSUPPORTED;
  if (workspace && ((uintptr_t)workspace & 255u)) return VSA_ERR_UNSUPPORTED;
  const size_t have = workspace && workspace_bytes ? *workspace_bytes : 0;
  return from_hip(vsa::launch_attn_fwd(a, workspace, have, stream));
}

vsa_status vsa_block_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                     const void* dout, const float* lse, float* dq, float* dk, float* dv,
                                     int32_t dtype, int64_t batch, int32_t heads, int32_t head_dim, int64_t nq,
                                     int64_t nk, int32_t block_q, int32_t block_k, const int32_t* row_ptr,
                                     const int32_t* col_idx, int32_t n_slabs, float scale, void* workspace,
                                     size_t* workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !o || !dout || !lse || !row_ptr || !col_idx) return VSA_ERR_NULL;
  vsa_status st = check_tokens(dtype, batch, heads, head_dim, nq, nk, block_q, block_k);
  if (st != VSA_OK) return st;
  if (n_slabs != 1 && (int64_t)n_slabs != batch * heads) return VSA_ERR_PARAM;
  if (!(scale > 0.0f) || scale == INFINITY) return VSA_ERR_PARAM;
  const int64_t nbq = ceil_div(nq, block_q), nbk = ceil_div(nk, block_k);
  if ((int64_t)n_slabs * nbq * nbk > kI32Max || batch * heads * nq > kI32Max) return VSA_ERR_SHAPE;
  if (dtype == VSA_BF16 && !bf16_rows_fit(heads, head_dim)) return VSA_ERR_UNSUPPORTED;
  vsa::AttnBwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, dtype, batch, heads, head_dim, nq, nk, block_q, block_k,
                     row_ptr, col_idx, n_slabs, scale};
  const size_t need = vsa::attn_bwd_workspace(a);
  if (!workspace) {
    if (!workspace_bytes) return VSA_ERR_NULL;
    *workspace_bytes = need;  // size query
    return VSA_OK;
  }
  if (!workspace_bytes || *workspace_bytes < need) return VSA_ERR_CAPACITY;
  if (!dq || !dk || !dv) return VSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || ((uintptr_t)workspace & 255u))
    return VSA_ERR_UNSUPPORTED;
  return from_hip(vsa::launch_attn_bwd(a, workspace, stream));
}

}  // extern "C"

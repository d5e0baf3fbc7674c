// Internal declarations shared by the HIP sources of libvsa (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsa {

constexpr int kWave = 64;

// ---------------------------------------------------------------- wave helpers
__device__ inline int lane_id() { return __lane_id(); }

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ inline int wave_inclusive_scan(int x) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int y = __shfl_up(x, o, kWave);
    if (l >= o) x += y;
  }
  return x;
}

// Number of set bits of a 64-bit ballot strictly below this lane.
__device__ inline int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// ------------------------------------------------------------- host launchers
hipError_t launch_tile_reorder(const void* src, void* dst, int64_t batch, int T, int H, int W,
                               int tt, int th, int tw, int64_t row_bytes, int inverse,
                               hipStream_t stream);

hipError_t launch_mask_sta(int NT, int NH, int NW, int ht, int hh, int hw, int32_t* row_ptr,
                           int32_t* col_idx, hipStream_t stream);

hipError_t launch_mask_radial(int T, int S, int block, int32_t* row_ptr, int32_t* col_idx,
                              hipStream_t stream);

// In-place: row_ptr[1..n] holds per-row counts on entry, absolute offsets on exit.
hipError_t launch_counts_to_offsets(int32_t* row_ptr, int64_t n_rows, hipStream_t stream);

// STA with one window per head: half-widths per head, slabs in (batch, head) order.
constexpr int kMaxStaHeads = 256;
struct StaHeads {
  int NT, NH, NW, heads;
  int16_t half[kMaxStaHeads][3];
};
hipError_t launch_mask_sta_heads(const StaHeads& p, int64_t n_rows, int32_t* row_ptr, int32_t* col_idx,
                                 hipStream_t stream);

// Union of two CSR masks over n_qblocks rows per slab; a one-slab mask is shared.
struct UnionArgs {
  const int32_t *rp_a, *ci_a, *rp_b, *ci_b;
  int64_t slabs_a, slabs_b, n_qblocks;
};
hipError_t launch_mask_union(const UnionArgs& u, int64_t n_rows, int32_t* row_ptr, int32_t* col_idx,
                             hipStream_t stream);

// SICS block scores of x [batch, n, heads, D] -> scores [batch, heads, ceil(n / block)] fp64.
hipError_t launch_block_sics(const void* x, int bf16, int64_t batch, int heads, int D, int64_t n, int block,
                             double* scores, hipStream_t stream);

// KV-cache compaction: slot map per slab, gather into the compact cache, mask remap.
hipError_t launch_kv_plan(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_slabs, int64_t n_qblocks,
                          int n_kblocks, int tail, int32_t* slot, int32_t* info, hipStream_t stream);
hipError_t launch_kv_gather(const void* x, int64_t batch, int64_t nk, int block_k, int heads, int row_vec,
                            int n_kblocks, const int32_t* slot, int64_t n_slabs, void* out, int64_t n_out,
                            hipStream_t stream);
hipError_t launch_mask_remap(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_qblocks,
                             const int32_t* slot, int n_kblocks, int64_t n_slabs, int32_t* col_out,
                             hipStream_t stream);

struct NablaArgs {
  const void* q;
  const void* k;
  int dtype;
  int64_t batch;
  int heads, head_dim;
  int64_t nq, nk;
  int block_q, block_k;
  double scale;
  double threshold;
  int topk;
  int n_forced;
  const int32_t* forced;  // host
  int32_t* row_ptr;
  int32_t* col_idx;
  void* workspace;
};
size_t nabla_workspace_bytes(int64_t batch, int heads, int head_dim, int64_t nq, int64_t nk,
                             int block_q, int block_k);
// Mean of the valid rows of each block: x [batch, n, heads, D] -> out [batch, nb, heads, D] fp64
// (the pooling pass of the NABLA mask on one tensor).
hipError_t launch_block_pool(const void* x, int bf16, int64_t batch, int heads, int D, int64_t n, int block,
                             double* out, hipStream_t stream);
hipError_t launch_mask_nabla(const NablaArgs& a, hipStream_t stream);

// Work items of the attention kernels are dealt to the 8 XCDs either as contiguous ranges
// (0) or in runs of this many consecutive items per XCD (see the kernels' Work).  Runs pay
// when one head's K and V take at least half the 256 MB Infinity Cache: with ranges, the XCDs
// work on 8 different heads at once and their K and V cannot share that cache; with runs, all
// XCDs work on neighbouring items of one head.  Measured bit for bit: the radial forward
// 520.8 -> 500.6 ms and backward 2,207.7 -> 2,079.3 ms (230 MB per head); sta (59 MB per head,
// whose windows stay local to each XCD's L2) 0.5-0.9% slower with runs, so it keeps ranges.
inline int xcd_run(int64_t nk, int head_dim, int dtype_bytes) {
  return 2 * nk * (int64_t)head_dim * dtype_bytes >= (int64_t)128 << 20 ? 32 : 0;
}

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int dtype;
  int64_t batch;
  int heads, head_dim;
  int64_t nq, nk;
  int block_q, block_k;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int n_slabs;
  float scale;
  // tiled: q, k, v, o and lse are in raster order of a T x H x W grid whose tt x th x tw
  // tiles, in tile-major order, are the attention blocks (block_q = block_k = tt th tw)
  int tiled = 0;
  int H = 0, W = 0, tt = 0, th = 0, tw = 0;
  // grouped query blocks: a group's blocks lie group_stride blocks apart (1: consecutive)
  int group_stride = 1;
};
// How a tiled forward maps its 64-row copy tiles (0: the tile shape is not supported):
// the tile's h-w plane must be a multiple of 64 tokens with tw dividing 64 or a multiple
// of 64, or divide 64.
int tiling_mode(int th, int tw);
// The tiled forward walks at most this many 64-token copy tiles per tile (tiles of up to
// 4096 tokens); larger tiles are not supported.
constexpr int kTiledMaxCopyTiles = 64;
// Largest lane part (rows after the copy tile's first token) of a 64-row copy tile of a
// supported tile shape (-1 if unsupported); the bf16 kernel adds it as a 32-bit offset.
int64_t tiling_lane_span(int H, int W, int th, int tw);
// Workspace the bf16 forward uses for grouped query blocks (0 if none); without it the
// call runs ungrouped.
// Workspace bytes of the fastest plan (union lists, split partials, packed V^T), and the
// least with which the call still runs grouped / split as planned (no packed V^T).
size_t attn_fwd_workspace(const AttnArgs& a);
size_t attn_fwd_workspace_min(const AttnArgs& a);
hipError_t launch_attn_fwd(const AttnArgs& a, void* workspace, size_t workspace_bytes, hipStream_t stream);

struct AttnBwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float* lse;
  float *dq, *dk, *dv;
  int dtype;
  int64_t batch;
  int heads, head_dim;
  int64_t nq, nk;
  int block_q, block_k;
  const int32_t *row_ptr, *col_idx;
  int n_slabs;
  float scale;
};
size_t attn_bwd_workspace(const AttnBwdArgs& a);
hipError_t launch_attn_bwd(const AttnBwdArgs& a, void* workspace, hipStream_t stream);

}  // namespace vsa

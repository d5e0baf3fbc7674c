// KV-cache compaction (Sparse Forcing summary, gist.science/ja/paper/2604.21221,
// parts 2-3): keep only the key blocks a (batch, head) still attends to, packed
// into a smaller cache with the same [batch, tokens, heads, head_dim] layout, and
// rewrite the mask onto the packed slots.
//
//   plan    one workgroup per slab marks the blocks any row of the slab keeps, then
//           ranks the kept full blocks (slot = rank, -1 = dropped); a kept ragged
//           last block takes the shared tail slot = the largest full count over
//           the slabs, filled in by a second, single-workgroup pass;
//   gather  one workgroup per (batch, block, token chunk) copies the block's token
//           rows, 16 bytes per lane, for the heads that keep it, to their slots;
//   remap   one wave per mask row rewrites its columns to slots (order is kept,
//           the slot map being increasing).
#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kPlanThreads = 1024;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Exclusive prefix sum of one value per thread over the workgroup; *total gets the sum.
// Every thread of the workgroup must call it.
__device__ int block_exclusive_scan(int f, int* total) {
  __shared__ int wave_tot[kPlanThreads / kWave];
  const int t = threadIdx.x, l = lane_id(), w = t / kWave;
  const int incl = wave_inclusive_scan(f);
  if (l == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  if (w == 0) {
    int x = l < kPlanThreads / kWave ? wave_tot[l] : 0;
    x = wave_inclusive_scan(x);
    if (l < kPlanThreads / kWave) wave_tot[l] = x;
  }
  __syncthreads();
  const int excl = (w > 0 ? wave_tot[w - 1] : 0) + incl - f;
  *total = wave_tot[kPlanThreads / kWave - 1];
  __syncthreads();
  return excl;
}

// slot[s][j] = rank of block j among the full blocks slab s keeps (-1: dropped); a kept
// ragged tail is marked -2 until the finishing pass gives it the shared tail slot.
// info[2 + s] = full blocks kept by slab s; info[2 + n_slabs + s] = 1 if it keeps the tail.
__global__ __launch_bounds__(kPlanThreads) void kv_plan_kernel(const int32_t* __restrict__ row_ptr,
                                                               const int32_t* __restrict__ col_idx,
                                                               int64_t n_qblocks, int n_kblocks, int tail,
                                                               int32_t* __restrict__ slot,
                                                               int32_t* __restrict__ info, int64_t n_slabs) {
  const int64_t s = blockIdx.x;
  int32_t* sl = slot + s * n_kblocks;
  for (int j = threadIdx.x; j < n_kblocks; j += kPlanThreads) sl[j] = 0;
  __threadfence_block();
  __syncthreads();
  const int32_t e0 = row_ptr[s * n_qblocks], e1 = row_ptr[(s + 1) * n_qblocks];
  for (int32_t e = e0 + threadIdx.x; e < e1; e += kPlanThreads) sl[col_idx[e]] = 1;  // same value: benign
  __threadfence_block();
  __syncthreads();
  const int keeps_tail = tail >= 0 ? sl[tail] : 0;
  int n_full = 0;
  for (int base = 0; base < n_kblocks; base += kPlanThreads) {
    const int j = base + threadIdx.x;
    const int f = j < n_kblocks && j != tail ? sl[j] : 0;
    int chunk = 0;
    const int excl = block_exclusive_scan(f, &chunk);
    if (j < n_kblocks) sl[j] = f ? n_full + excl : -1;
    n_full += chunk;
  }
  __threadfence_block();
  __syncthreads();
  if (threadIdx.x == 0) {
    if (tail >= 0) sl[tail] = keeps_tail ? -2 : -1;
    info[2 + s] = n_full;
    info[2 + n_slabs + s] = keeps_tail;
  }
}

// info[0] = largest full count over the slabs (= the tail slot), info[1] = 1 if any
// slab keeps the tail; then the tail markers become that slot.
__global__ __launch_bounds__(kPlanThreads) void kv_plan_finish_kernel(int64_t n_slabs, int n_kblocks, int tail,
                                                                      int32_t* __restrict__ slot,
                                                                      int32_t* __restrict__ info) {
  __shared__ int red_max[kPlanThreads / kWave], red_any[kPlanThreads / kWave];
  int m = 0, any = 0;
  for (int64_t s = threadIdx.x; s < n_slabs; s += kPlanThreads) {
    m = max(m, info[2 + s]);
    any |= info[2 + n_slabs + s];
  }
  for (int o = kWave / 2; o > 0; o >>= 1) {
    m = max(m, __shfl_xor(m, o, kWave));
    any |= __shfl_xor(any, o, kWave);
  }
  if (lane_id() == 0) red_max[threadIdx.x / kWave] = m, red_any[threadIdx.x / kWave] = any;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kPlanThreads / kWave; ++i) m = max(m, red_max[i]), any |= red_any[i];
    red_max[0] = m;
    info[0] = m;
    info[1] = any;
  }
  __syncthreads();
  if (tail < 0) return;
  const int tslot = red_max[0];
  for (int64_t s = threadIdx.x; s < n_slabs; s += kPlanThreads)
    if (slot[s * n_kblocks + tail] == -2) slot[s * n_kblocks + tail] = tslot;
}

// grid: x = (key block, chunk of 8 of its tokens), y = batch.  Writes past n_out (a
// compact size smaller than the plan's) are dropped rather than made.
constexpr int kGatherThreads = 256;
constexpr int kTokensPerGroup = 8;
__global__ __launch_bounds__(kGatherThreads) void kv_gather_kernel(const u32x4* __restrict__ x, int64_t nk,
                                                                   int block_k, int chunks, int heads,
                                                                   int vec_per_head, int n_kblocks,
                                                                   const int32_t* __restrict__ slot,
                                                                   int64_t n_slabs, u32x4* __restrict__ out,
                                                                   int64_t n_out) {
  const int j = blockIdx.x / chunks, chunk = blockIdx.x % chunks;
  const int64_t b = blockIdx.y;
  const int vpr = heads * vec_per_head;  // 16-byte vectors per token row
  const int64_t t_lo = (int64_t)j * block_k + (int64_t)chunk * kTokensPerGroup;
  const int64_t t_hi = min(min(t_lo + kTokensPerGroup, (int64_t)(j + 1) * block_k), nk);
  for (int64_t idx = threadIdx.x; idx < (t_hi - t_lo) * vpr; idx += kGatherThreads) {
    const int64_t t = t_lo + idx / vpr;
    const int v = (int)(idx % vpr), h = v / vec_per_head;
    const int64_t s = n_slabs == 1 ? 0 : b * heads + h;
    const int32_t c = slot[s * n_kblocks + j];
    if (c < 0) continue;
    const int64_t dst = (int64_t)c * block_k + (t - (int64_t)j * block_k);
    if (dst >= n_out) continue;
    out[(b * n_out + dst) * vpr + v] = __builtin_nontemporal_load(&x[(b * nk + t) * vpr + v]);
  }
}

constexpr int kRowsPerBlock = 4;
__global__ __launch_bounds__(kRowsPerBlock * kWave) void mask_remap_kernel(const int32_t* __restrict__ row_ptr,
                                                                           const int32_t* __restrict__ col_idx,
                                                                           int64_t n_rows, int64_t n_qblocks,
                                                                           const int32_t* __restrict__ slot,
                                                                           int n_kblocks, int64_t n_slabs,
                                                                           int32_t* __restrict__ col_out) {
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (r >= n_rows) return;
  const int64_t s = n_slabs == 1 ? 0 : r / n_qblocks;
  const int32_t* sl = slot + s * n_kblocks;
  for (int32_t e = row_ptr[r] + lane_id(); e < row_ptr[r + 1]; e += kWave) col_out[e] = sl[col_idx[e]];
}

}  // namespace

hipError_t launch_kv_plan(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_slabs, int64_t n_qblocks,
                          int n_kblocks, int tail, int32_t* slot, int32_t* info, hipStream_t stream) {
  hipLaunchKernelGGL(kv_plan_kernel, dim3((unsigned)n_slabs), dim3(kPlanThreads), 0, stream, row_ptr, col_idx,
                     n_qblocks, n_kblocks, tail, slot, info, n_slabs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv_plan_finish_kernel, dim3(1), dim3(kPlanThreads), 0, stream, n_slabs, n_kblocks, tail,
                     slot, info);
  return hipGetLastError();
}

hipError_t launch_kv_gather(const void* x, int64_t batch, int64_t nk, int block_k, int heads, int row_vec,
                            int n_kblocks, const int32_t* slot, int64_t n_slabs, void* out, int64_t n_out,
                            hipStream_t stream) {
  const int chunks = (block_k + kTokensPerGroup - 1) / kTokensPerGroup;
  const dim3 grid((unsigned)((int64_t)n_kblocks * chunks), (unsigned)batch);
  hipLaunchKernelGGL(kv_gather_kernel, grid, dim3(kGatherThreads), 0, stream, (const u32x4*)x, nk, block_k,
                     chunks, heads, row_vec / heads, n_kblocks, slot, n_slabs, (u32x4*)out, n_out);
  return hipGetLastError();
}

hipError_t launch_mask_remap(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_qblocks,
                             const int32_t* slot, int n_kblocks, int64_t n_slabs, int32_t* col_out,
                             hipStream_t stream) {
  const dim3 grid((unsigned)((n_rows + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL(mask_remap_kernel, grid, dim3(kRowsPerBlock * kWave), 0, stream, row_ptr, col_idx, n_rows,
                     n_qblocks, slot, n_kblocks, n_slabs, col_out);
  return hipGetLastError();
}

}  // namespace vsa

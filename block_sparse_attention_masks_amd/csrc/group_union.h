// Union lists for grouped blocks, shared by the forward (G query blocks per workgroup,
// over the CSR rows) and the backward (G key blocks per workgroup, over the CSC columns).
#pragma once

#include "vsa_internal.h"

namespace vsa {
namespace {

// Lists `ptr` / `idx` (CSR rows, or CSC columns) hold n_per_slab lists per slab, each
// ascending.  Group g of a slab joins G lists `stride` apart: with g = c stride + j, lists
// c stride G + j + i stride for i < G (stride 1: lists g G .. g G + G - 1).  One wave per (slab,
// group): lane r < G walks list r of the group; each step takes the smallest index any
// lane still holds (a wave minimum), records the lanes holding it as the entry's mask, and
// advances them.  The union for u = slab * n_groups + g is written at out_idx[u * cap ..]
// and out_mask[u * cap ..], its length to out_cnt[u].
constexpr int kUnionWaves = 4;
__global__ __launch_bounds__(kUnionWaves * kWave) void group_union_kernel(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx, int n_per_slab, int64_t n_lists, int G,
    int n_groups, int stride, int cap, int32_t* __restrict__ out_idx, int32_t* __restrict__ out_mask,
    int32_t* __restrict__ out_cnt) {
  const int64_t u = (int64_t)blockIdx.x * kUnionWaves + threadIdx.x / kWave;
  if (u >= n_lists) return;
  const int l = lane_id();
  const int64_t slab = u / n_groups;
  const int gi = (int)(u % n_groups);
  const int r = (gi / stride) * stride * G + gi % stride + l * stride;
  int32_t e = 0, e1 = 0;
  if (l < G && r < n_per_slab) {
    e = ptr[slab * n_per_slab + r];
    e1 = ptr[slab * n_per_slab + r + 1];
  }
  int32_t* oc = out_idx + u * cap;
  int32_t* om = out_mask + u * cap;
  int n = 0;
  while (true) {
    const int32_t val = e < e1 ? idx[e] : INT32_MAX;
    int32_t m = val;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) m = min(m, __shfl_xor(m, o, kWave));
    if (m == INT32_MAX || n >= cap) break;  // cap: lists hold distinct indices below it
    const uint64_t bits = __ballot(val == m);
    if (l == 0) {
      oc[n] = m;
      om[n] = (int32_t)bits;
    }
    if (val == m) ++e;
    ++n;
  }
  if (l == 0) out_cnt[u] = n;
}

// The same lists from bitmaps, when the G bitmaps of cap bits fit in LDS: the wave sets bit j
// of row r's bitmap for every entry j of list r (LDS atomic OR), then sweeps j = 0 .. cap - 1,
// 64 at a time: lane j's mask collects bit j of the G bitmaps, and the lanes with a nonzero
// mask write their (j, mask) in ascending order (ballot and lane prefix count).  The output is
// the walk's, entry for entry; its cost is the lists' entries plus cap / 64 steps, where the
// walk takes one wave minimum per union entry.
constexpr int kUnionBitmapWords = 4096;  // per wave: 16 KB of the workgroup's 64 KB
__global__ __launch_bounds__(kUnionWaves * kWave) void group_union_bitmap_kernel(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx, int n_per_slab, int64_t n_lists, int G,
    int n_groups, int stride, int cap, int words, int32_t* __restrict__ out_idx, int32_t* __restrict__ out_mask,
    int32_t* __restrict__ out_cnt) {
  extern __shared__ uint32_t union_bitmaps[];
  const int wv = threadIdx.x / kWave;
  const int64_t u = (int64_t)blockIdx.x * kUnionWaves + wv;
  if (u >= n_lists) return;  // waves work alone: no workgroup barrier below
  const int l = lane_id();
  uint32_t* bm = union_bitmaps + wv * G * words;
  for (int i = l; i < G * words; i += kWave) bm[i] = 0u;
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the clears have landed before any OR
  __builtin_amdgcn_wave_barrier();
  const int64_t slab = u / n_groups;
  const int gi = (int)(u % n_groups);
  for (int r = 0; r < G; ++r) {
    const int row = (gi / stride) * stride * G + gi % stride + r * stride;
    if (row >= n_per_slab) break;  // rows ascend with r
    const int32_t e0 = ptr[slab * n_per_slab + row], e1 = ptr[slab * n_per_slab + row + 1];
    for (int32_t e = e0 + l; e < e1; e += kWave) {
      const int32_t j = idx[e];
      atomicOr(&bm[r * words + (j >> 5)], 1u << (j & 31));
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // every OR has landed before the sweep reads
  __builtin_amdgcn_wave_barrier();
  int32_t* oc = out_idx + u * cap;
  int32_t* om = out_mask + u * cap;
  int n = 0;
  for (int j0 = 0; j0 < cap; j0 += kWave) {
    const int j = j0 + l;
    uint32_t m = 0;
    if (j < cap)
      for (int r = 0; r < G; ++r) m |= ((bm[r * words + (j >> 5)] >> (j & 31)) & 1u) << r;
    const uint64_t bits = __ballot(m != 0);
    const int pos = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
    if (m != 0) {
      oc[pos] = j;
      om[pos] = (int32_t)m;
    }
    n += __builtin_popcountll(bits);
  }
  if (l == 0) out_cnt[u] = n;
}

// Union lists of n_lists groups: the bitmap kernel when a wave's G bitmaps of cap bits fit its
// share of LDS, else the walk.
inline hipError_t launch_group_union(const int32_t* ptr, const int32_t* idx, int n_per_slab, int64_t n_lists, int G,
                                     int n_groups, int stride, int cap, int32_t* out_idx, int32_t* out_mask,
                                     int32_t* out_cnt, hipStream_t stream) {
  const dim3 grid((unsigned)((n_lists + kUnionWaves - 1) / kUnionWaves)), block(kUnionWaves * kWave);
  const int words = (cap + 31) / 32;
  if ((int64_t)G * words <= kUnionBitmapWords) {
    hipLaunchKernelGGL(group_union_bitmap_kernel, grid, block, kUnionWaves * G * words * sizeof(uint32_t), stream,
                       ptr, idx, n_per_slab, n_lists, G, n_groups, stride, cap, words, out_idx, out_mask, out_cnt);
  } else {
    hipLaunchKernelGGL(group_union_kernel, grid, block, 0, stream, ptr, idx, n_per_slab, n_lists, G, n_groups, stride,
                       cap, out_idx, out_mask, out_cnt);
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace vsa

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

}  // namespace
}  // namespace vsa

// Mask composition: STA with a window per head, and the union of two CSR masks.
//
// Both are written as count -> scan -> fill over all output rows, like the other
// masks: a pass writes the number of kept key blocks per row into row_ptr[1..n],
// the shared scan turns the counts into offsets, and a fill pass writes each
// row's columns in ascending order.
#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kThreadsPerBlock = 256;

// ------------------------------------------------------------ per-head STA
// Number of tiles within +-h of c on an axis of n tiles (window clipped at the border).
__device__ inline int span(int c, int n, int h) { return min(n - 1, c + h) - max(0, c - h) + 1; }

// Row r of the output is tile i = r % n of slab r / n; the slab's head is slab % heads.
__global__ __launch_bounds__(kThreadsPerBlock) void sta_heads_count_kernel(StaHeads p, int64_t n_rows,
                                                                          int32_t* row_ptr) {
  const int64_t r = (int64_t)blockIdx.x * kThreadsPerBlock + threadIdx.x;
  if (r >= n_rows) return;
  const int n = p.NT * p.NH * p.NW;
  const int h = (int)((r / n) % p.heads), i = (int)(r % n);
  const int ct = i / (p.NH * p.NW), ch = (i / p.NW) % p.NH, cw = i % p.NW;
  row_ptr[r + 1] = span(ct, p.NT, p.half[h][0]) * span(ch, p.NH, p.half[h][1]) * span(cw, p.NW, p.half[h][2]);
}

__global__ __launch_bounds__(kThreadsPerBlock) void sta_heads_fill_kernel(StaHeads p, int64_t n_rows,
                                                                         const int32_t* row_ptr,
                                                                         int32_t* col_idx) {
  const int64_t r = (int64_t)blockIdx.x * kThreadsPerBlock + threadIdx.x;
  if (r >= n_rows) return;
  const int n = p.NT * p.NH * p.NW;
  const int h = (int)((r / n) % p.heads), i = (int)(r % n);
  const int ht = p.half[h][0], hh = p.half[h][1], hw = p.half[h][2];
  const int ct = i / (p.NH * p.NW), ch = (i / p.NW) % p.NH, cw = i % p.NW;
  int32_t* out = col_idx + row_ptr[r];
  for (int jt = max(0, ct - ht); jt <= min(p.NT - 1, ct + ht); ++jt)
    for (int jh = max(0, ch - hh); jh <= min(p.NH - 1, ch + hh); ++jh)
      for (int jw = max(0, cw - hw); jw <= min(p.NW - 1, cw + hw); ++jw)
        *out++ = (jt * p.NH + jh) * p.NW + jw;
}

// ------------------------------------------------------------------ union
constexpr int kRowsPerBlock = 4;  // one wave per output row

// First index of a[0..n) (ascending) holding a value >= x.
__device__ inline int lower_bound(const int32_t* a, int n, int32_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

struct RowPair {
  const int32_t *a, *b;
  int na, nb;
};

__device__ inline RowPair row_pair(const UnionArgs& u, int64_t r) {
  const int64_t s = r / u.n_qblocks, i = r % u.n_qblocks;
  const int64_t ra = (u.slabs_a > 1 ? s : 0) * u.n_qblocks + i;
  const int64_t rb = (u.slabs_b > 1 ? s : 0) * u.n_qblocks + i;
  const int32_t a0 = u.rp_a[ra], b0 = u.rp_b[rb];
  return {u.ci_a + a0, u.ci_b + b0, u.rp_a[ra + 1] - a0, u.rp_b[rb + 1] - b0};
}

// |A u B| = |A| + |B| - |A n B|; each lane looks its A entries up in B.
__global__ __launch_bounds__(kRowsPerBlock * kWave) void union_count_kernel(UnionArgs u, int64_t n_rows,
                                                                            int32_t* row_ptr) {
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (r >= n_rows) return;
  const RowPair p = row_pair(u, r);
  int dup = 0;
  for (int e = lane_id(); e < p.na; e += kWave) {
    const int32_t x = p.a[e];
    const int j = lower_bound(p.b, p.nb, x);
    dup += j < p.nb && p.b[j] == x;
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) dup += __shfl_xor(dup, o, kWave);
  if (lane_id() == 0) row_ptr[r + 1] = p.na + p.nb - dup;
}

// In the ascending union, x sits after every smaller entry of either row, counting
// the entries the rows share once: slot(x) = #(A < x) + #(B < x) - #(A n B < x).  For
// A[e] that is e + #(B < A[e]) - (shared entries among A[0..e)); B[e], when not in A,
// goes to e + #(A < B[e]) - (shared entries among B[0..e)).  The shared counts are a
// ballot prefix over each 64-entry chunk plus a running carry.
__global__ __launch_bounds__(kRowsPerBlock * kWave) void union_fill_kernel(UnionArgs u, int64_t n_rows,
                                                                           const int32_t* row_ptr,
                                                                           int32_t* col_idx) {
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (r >= n_rows) return;
  const RowPair p = row_pair(u, r);
  int32_t* out = col_idx + row_ptr[r];
  const int l = lane_id();
  int carry = 0;
  for (int base = 0; base < p.na; base += kWave) {
    const int e = base + l;
    int32_t x = 0;
    int slot = 0, shared = 0;
    if (e < p.na) {
      x = p.a[e];
      const int j = lower_bound(p.b, p.nb, x);
      shared = j < p.nb && p.b[j] == x;
      slot = e + j;
    }
    const uint64_t m = __ballot(shared);
    if (e < p.na) out[slot - carry - lanes_below(m)] = x;
    carry += __popcll(m);
  }
  carry = 0;
  for (int base = 0; base < p.nb; base += kWave) {
    const int e = base + l;
    int32_t x = 0;
    int slot = 0, shared = 0;
    if (e < p.nb) {
      x = p.b[e];
      const int j = lower_bound(p.a, p.na, x);
      shared = j < p.na && p.a[j] == x;
      slot = e + j;
    }
    const uint64_t m = __ballot(shared);
    if (e < p.nb && !shared) out[slot - carry - lanes_below(m)] = x;
    carry += __popcll(m);
  }
}

}  // namespace

hipError_t launch_mask_sta_heads(const StaHeads& p, int64_t n_rows, int32_t* row_ptr, int32_t* col_idx,
                                 hipStream_t stream) {
  const dim3 grid((unsigned)((n_rows + kThreadsPerBlock - 1) / kThreadsPerBlock));
  hipLaunchKernelGGL(sta_heads_count_kernel, grid, dim3(kThreadsPerBlock), 0, stream, p, n_rows, row_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_counts_to_offsets(row_ptr, n_rows, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(sta_heads_fill_kernel, grid, dim3(kThreadsPerBlock), 0, stream, p, n_rows, row_ptr,
                     col_idx);
  return hipGetLastError();
}

hipError_t launch_mask_union(const UnionArgs& u, int64_t n_rows, int32_t* row_ptr, int32_t* col_idx,
                             hipStream_t stream) {
  const dim3 grid((unsigned)((n_rows + kRowsPerBlock - 1) / kRowsPerBlock)), threads(kRowsPerBlock * kWave);
  hipLaunchKernelGGL(union_count_kernel, grid, threads, 0, stream, u, n_rows, row_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_counts_to_offsets(row_ptr, n_rows, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(union_fill_kernel, grid, threads, 0, stream, u, n_rows, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace vsa

// Static block masks (STA tile window, radial energy decay) and the CSR build
// shared with the dynamic masks.
//
// Every mask is written as count -> scan -> fill: a pass computes the number of
// kept key blocks per row into row_ptr[1..n], a scan turns counts into absolute
// offsets, and a fill pass writes each row's kept columns in ascending order.
// The radial passes use one wave per query block: each lane tests key blocks,
// a ballot collects the kept ones and mbcnt gives each lane its write slot.
#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kScanThreads = 1024;

// In-place inclusive scan of data[0..n) by one 1024-thread workgroup.
__device__ void block_inclusive_scan(int32_t* data, int64_t n) {
  __shared__ int32_t wave_sums[kScanThreads / kWave];
  __shared__ int32_t carry_s;
  const int t = threadIdx.x, l = lane_id(), w = t / kWave;
  if (t == 0) carry_s = 0;
  __syncthreads();
  for (int64_t base = 0; base < n; base += kScanThreads) {
    const int64_t i = base + t;
    int x = i < n ? data[i] : 0;
    int incl = wave_inclusive_scan(x);
    if (l == kWave - 1) wave_sums[w] = incl;
    __syncthreads();
    if (w == 0) {
      int s = l < kScanThreads / kWave ? wave_sums[l] : 0;
      s = wave_inclusive_scan(s);
      if (l < kScanThreads / kWave) wave_sums[l] = s;
    }
    __syncthreads();
    const int carry = carry_s;
    const int before = (w > 0 ? wave_sums[w - 1] : 0) + carry;
    if (i < n) data[i] = incl + before;
    __syncthreads();
    if (t == kScanThreads - 1) carry_s = carry + wave_sums[kScanThreads / kWave - 1];
    __syncthreads();
  }
}

__global__ __launch_bounds__(kScanThreads) void counts_to_offsets_kernel(int32_t* row_ptr,
                                                                         int64_t n) {
  if (threadIdx.x == 0) row_ptr[0] = 0;
  block_inclusive_scan(row_ptr + 1, n);
}

// ------------------------------------------------------------------------ STA
// Number of tiles within +-h of c on an axis of n tiles (window clipped at the border).
__device__ inline int clipped_span(int c, int n, int h) {
  return min(n - 1, c + h) - max(0, c - h) + 1;
}

__global__ __launch_bounds__(kScanThreads) void mask_sta_kernel(int NT, int NH, int NW, int ht,
                                                                int hh, int hw,
                                                                int32_t* row_ptr,
                                                                int32_t* col_idx) {
  const int n = NT * NH * NW;
  for (int i = threadIdx.x; i < n; i += kScanThreads) {
    const int ct = i / (NH * NW), ch = (i / NW) % NH, cw = i % NW;
    row_ptr[i + 1] = clipped_span(ct, NT, ht) * clipped_span(ch, NH, hh) * clipped_span(cw, NW, hw);
  }
  if (threadIdx.x == 0) row_ptr[0] = 0;
  __threadfence_block();
  __syncthreads();
  block_inclusive_scan(row_ptr + 1, n);
  __threadfence_block();
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kScanThreads) {
    const int ct = i / (NH * NW), ch = (i / NW) % NH, cw = i % NW;
    int out = row_ptr[i];
    for (int jt = max(0, ct - ht); jt <= min(NT - 1, ct + ht); ++jt)
      for (int jh = max(0, ch - hh); jh <= min(NH - 1, ch + hh); ++jh)
        for (int jw = max(0, cw - hw); jw <= min(NW - 1, cw + hw); ++jw)
          col_idx[out++] = (jt * NH + jh) * NW + jw;
  }
}

// --------------------------------------------------------------------- radial
struct Radial {
  int T, S, block, N, nb;
};

// Block pair test.  For every (query frame f, key frame g) pair that the two
// blocks touch, the blocks hold in-frame index runs [qa, qb] and [ka, kb]; the
// closest token pair is `gap` apart.  The pair is kept iff d = |f - g| <= 1 or
// gap * 2^floor(log2 d) < S, i.e. gap <= (S - 1) >> floor(log2 d).
__device__ inline bool radial_pair(int I, int J, const Radial& p) {
  const int q0 = I * p.block, q1 = min(q0 + p.block, p.N) - 1;
  const int k0 = J * p.block, k1 = min(k0 + p.block, p.N) - 1;
  const int f0 = q0 / p.S, f1 = q1 / p.S, g0 = k0 / p.S, g1 = k1 / p.S;
  // Any two frames at distance <= 1 make the pair dense.
  if (g0 <= f1 + 1 && f0 <= g1 + 1) return true;
  for (int f = f0; f <= f1; ++f) {
    const int qa = max(q0, f * p.S) - f * p.S, qb = min(q1, f * p.S + p.S - 1) - f * p.S;
    for (int g = g0; g <= g1; ++g) {
      const int ka = max(k0, g * p.S) - g * p.S, kb = min(k1, g * p.S + p.S - 1) - g * p.S;
      const int d = f > g ? f - g : g - f;          // >= 2 here
      const int r = 31 - __builtin_clz((unsigned)d);  // floor(log2 d)
      const int gap = max(0, max(ka - qb, qa - kb));
      if (gap <= ((p.S - 1) >> r)) return true;
    }
  }
  return false;
}

constexpr int kRowsPerBlock = 4;  // one wave per row

__global__ __launch_bounds__(kRowsPerBlock * kWave) void radial_count_kernel(Radial p,
                                                                             int32_t* row_ptr) {
  const int I = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (I >= p.nb) return;
  int count = 0;
  for (int J0 = 0; J0 < p.nb; J0 += kWave) {
    const int J = J0 + lane_id();
    const bool keep = J < p.nb && radial_pair(I, J, p);
    count += __popcll(__ballot(keep));
  }
  if (lane_id() == 0) row_ptr[I + 1] = count;
}

__global__ __launch_bounds__(kRowsPerBlock * kWave) void radial_fill_kernel(Radial p,
                                                                            const int32_t* row_ptr,
                                                                            int32_t* col_idx) {
  const int I = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (I >= p.nb) return;
  int out = row_ptr[I];
  for (int J0 = 0; J0 < p.nb; J0 += kWave) {
    const int J = J0 + lane_id();
    const bool keep = J < p.nb && radial_pair(I, J, p);
    const uint64_t m = __ballot(keep);
    if (keep) col_idx[out + lanes_below(m)] = J;
    out += __popcll(m);
  }
}

}  // namespace

hipError_t launch_counts_to_offsets(int32_t* row_ptr, int64_t n_rows, hipStream_t stream) {
  hipLaunchKernelGGL(counts_to_offsets_kernel, dim3(1), dim3(kScanThreads), 0, stream, row_ptr,
                     n_rows);
  return hipGetLastError();
}

hipError_t launch_mask_sta(int NT, int NH, int NW, int ht, int hh, int hw, int32_t* row_ptr,
                           int32_t* col_idx, hipStream_t stream) {
  hipLaunchKernelGGL(mask_sta_kernel, dim3(1), dim3(kScanThreads), 0, stream, NT, NH, NW, ht, hh,
                     hw, row_ptr, col_idx);
  return hipGetLastError();
}

hipError_t launch_mask_radial(int T, int S, int block, int32_t* row_ptr, int32_t* col_idx,
                              hipStream_t stream) {
  Radial p{T, S, block, T * S, (T * S + block - 1) / block};
  const dim3 grid((p.nb + kRowsPerBlock - 1) / kRowsPerBlock), threads(kRowsPerBlock * kWave);
  hipLaunchKernelGGL(radial_count_kernel, grid, threads, 0, stream, p, row_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_counts_to_offsets(row_ptr, p.nb, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(radial_fill_kernel, grid, threads, 0, stream, p, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace vsa

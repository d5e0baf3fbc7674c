// Dynamic block mask from mean-pooled Q and K (NABLA explainer, aibr.jp/archives/
// 124678, sec. 3), and the anchor + recent + top-k variant used for an
// autoregressive chunk step (Sparse Forcing summary, gist.science/ja/paper/
// 2604.21221, part 2).
//
// Four passes, all in fp64 so that the decision matches a plain fp64 evaluation
// except where the cumulative mass sits within rounding of the threshold:
//   1. pool      -- per block, exact fp64 sums of the (bf16 or fp32) token rows,
//                   one division by the number of valid tokens.  HBM-bound: one
//                   workgroup streams a block's rows with 16-byte loads.
//   2. score     -- Z = Qp Kp^T * scale per (batch, head), 64x64 fp64 tiles.
//   3. select    -- one workgroup per row: softmax of Z (NABLA) or raw Z (top-k),
//                   bitonic sort in LDS by (value desc, block asc), fp64 running
//                   sum, cut; writes a bitmap row and the kept count.
//   4. CSR       -- counts -> offsets (shared scan), then bitmap -> ascending
//                   column lists, one wave per row.
#include <float.h>

#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxForced = 16;
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t qp, kp, z, bits, total;
};

Layout layout(int64_t bh, int D, int64_t nbq, int64_t nbk) {
  Layout L;
  const int64_t words = (nbk + 31) / 32;
  L.qp = 0;
  L.kp = L.qp + align_up(sizeof(double) * bh * nbq * D);
  L.z = L.kp + align_up(sizeof(double) * bh * nbk * D);
  L.bits = L.z + align_up(sizeof(double) * bh * nbq * nbk);
  L.total = L.bits + align_up(sizeof(uint32_t) * bh * nbq * words);
  return L;
}

// ------------------------------------------------------------------- 1. pool
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes read once: a streaming (nontemporal) load, which does not displace cached
// lines (≈8% faster for this single pass over Q and K than a plain load)
__device__ inline uint4 load_stream(const uint8_t* p) {
  const u32x4 r = __builtin_nontemporal_load((const u32x4*)p);
  return uint4{r.x, r.y, r.z, r.w};
}

// 8 consecutive elements of a row widened to fp64: 16 bytes of bf16, or 32 of fp32.
template <bool BF16>
struct Vec8 {
  uint4 a, c;
  __device__ void load(const uint8_t* p) {
    a = load_stream(p);
    if constexpr (!BF16) c = load_stream(p + 16);
  }
  __device__ void add_to(double* acc) const {
    if constexpr (BF16) {
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += (double)__uint_as_float(w[i] << 16);
        acc[2 * i + 1] += (double)__uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += (double)__uint_as_float(w[i]);
    }
  }
};

// grid: x = query blocks then key blocks, y = column slices of 8*blockDim.x elements,
// z = batch.  The host sizes blockDim.x so that the slices cover a row evenly.  Each lane
// keeps U rows' loads in flight; the element type is a template parameter so that the
// bf16 kernel holds only its own registers (and so keeps enough waves resident).
constexpr int kPoolMaxThreads = 512;
template <bool BF16>
__global__ __launch_bounds__(kPoolMaxThreads) void pool_kernel(const uint8_t* __restrict__ q,
                                                        const uint8_t* __restrict__ k,
                                                        int64_t nq, int64_t nk, int bq, int bk,
                                                        int nbq, int nbk, int heads, int D,
                                                        double* __restrict__ qp,
                                                        double* __restrict__ kp) {
  const bool isq = (int)blockIdx.x < nbq;
  const int blk = isq ? blockIdx.x : blockIdx.x - nbq;
  const int64_t n = isq ? nq : nk;
  const int bsz = isq ? bq : bk;
  const int nb = isq ? nbq : nbk;
  const uint8_t* src = isq ? q : k;
  double* dst = isq ? qp : kp;
  const int64_t b = blockIdx.z;
  const int hd = heads * D;
  const int vec = blockIdx.y * blockDim.x + threadIdx.x;  // 8-element vector index in a row
  if (vec * 8 >= hd) return;
  constexpr int esz = BF16 ? 2 : 4;
  const int64_t row_bytes = (int64_t)hd * esz;
  const int64_t t0 = (int64_t)blk * bsz, t1 = min(n, t0 + bsz);
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const uint8_t* p = src + (b * n + t0) * row_bytes + (int64_t)vec * 8 * esz;
  int64_t t = t0;
  constexpr int U = BF16 ? 16 : 8;
  for (; t + U <= t1; t += U) {
    Vec8<BF16> x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u].load(p + u * row_bytes);
#pragma unroll
    for (int u = 0; u < U; ++u) x[u].add_to(acc);
    p += U * row_bytes;
  }
  for (; t < t1; ++t) {
    Vec8<BF16> x;
    x.load(p);
    x.add_to(acc);
    p += row_bytes;
  }
  const double cnt = (double)(t1 - t0);
  const int e0 = vec * 8, h = e0 / D, d0 = e0 % D;   // D is a multiple of 8
  double* out = dst + (((b * heads + h) * nb) + blk) * D + d0;
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = acc[i] / cnt;
}

// ------------------------------------------------------------------ 2. score
constexpr int kTile = 64, kKc = 16;

__global__ __launch_bounds__(kThreads) void score_kernel(const double* __restrict__ qp,
                                                         const double* __restrict__ kp, int nbq,
                                                         int nbk, int D, double scale,
                                                         double* __restrict__ z) {
  __shared__ double As[kKc][kTile + 1];
  __shared__ double Bs[kKc][kTile + 1];
  const int64_t bh = blockIdx.z;
  const int i0 = blockIdx.y * kTile, j0 = blockIdx.x * kTile;
  const double* A = qp + bh * nbq * (int64_t)D;
  const double* B = kp + bh * nbk * (int64_t)D;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  double acc[4][4] = {};
  for (int d0 = 0; d0 < D; d0 += kKc) {
    for (int e = threadIdx.x; e < kTile * kKc; e += kThreads) {
      const int r = e / kKc, c = e % kKc;
      As[c][r] = (i0 + r < nbq) ? A[(int64_t)(i0 + r) * D + d0 + c] : 0.0;
      Bs[c][r] = (j0 + r < nbk) ? B[(int64_t)(j0 + r) * D + d0 + c] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kKc; ++c) {
      double a[4], bb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = As[c][ty + 16 * u];
        bb[u] = Bs[c][tx + 16 * u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fma(a[u], bb[v], acc[u][v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = i0 + ty + 16 * u, j = j0 + tx + 16 * v;
      if (i < nbq && j < nbk) z[(bh * nbq + i) * (int64_t)nbk + j] = acc[u][v] * scale;
    }
}

// ----------------------------------------------------------------- 3. select
struct Forced {
  int n;
  int lo[kMaxForced], hi[kMaxForced];
};

__device__ inline bool before(double ka, int ia, double kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__device__ double block_reduce(double x, bool is_max, double* red) {
  const int l = lane_id(), w = threadIdx.x / kWave;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const double y = __shfl_xor(x, o, kWave);
    x = is_max ? fmax(x, y) : x + y;
  }
  __syncthreads();
  if (l == 0) red[w] = x;
  __syncthreads();
  double r = red[0];
  for (int i = 1; i < kThreads / kWave; ++i) r = is_max ? fmax(r, red[i]) : r + red[i];
  return r;
}

// dynamic LDS: double key[SN], int idx[SN], uint32 bits[words]
__global__ __launch_bounds__(kThreads) void select_kernel(const double* __restrict__ z, int nbk,
                                                          int SN, double thr, int topk, Forced fc,
                                                          uint32_t* __restrict__ bitmap,
                                                          int32_t* __restrict__ row_ptr) {
  extern __shared__ double smem[];
  __shared__ double red[kThreads / kWave];
  __shared__ double tsum[kThreads / kWave];
  __shared__ int cut_s;
  double* key = smem;
  int* idx = (int*)(key + SN);
  const int words = (nbk + 31) / 32;
  uint32_t* bits = (uint32_t*)(idx + SN);
  const int64_t row = blockIdx.x;
  const double* zr = z + row * nbk;
  const int t = threadIdx.x;
  for (int w = t; w < words; w += kThreads) bits[w] = 0;
  if (t == 0) cut_s = SN;

  int n_cand = nbk;
  if (topk == 0) {
    double m = -DBL_MAX;
    for (int j = t; j < nbk; j += kThreads) m = fmax(m, zr[j]);
    m = block_reduce(m, true, red);
    double s = 0;
    for (int j = t; j < nbk; j += kThreads) {
      const double e = exp(zr[j] - m);
      key[j] = e;
      s += e;
    }
    s = block_reduce(s, false, red);   // contains a barrier: key[] is visible after it
    for (int j = t; j < SN; j += kThreads) {
      key[j] = j < nbk ? key[j] / s : -1.0;
      idx[j] = j;
    }
  } else {
    n_cand = nbk;
    for (int r = 0; r < fc.n; ++r) n_cand -= fc.hi[r] - fc.lo[r];  // ranges are disjoint
    for (int j = t; j < SN; j += kThreads) {
      bool forced = false;
      for (int r = 0; r < fc.n; ++r) forced |= (j >= fc.lo[r] && j < fc.hi[r]);
      key[j] = (j < nbk && !forced) ? zr[j] : -DBL_MAX;
      idx[j] = j;
    }
  }
  __syncthreads();

  // Bitonic sort of (key, idx) into `before` order.  Each thread takes whole pairs: pair q
  // of a stage joins i (q with a zero bit inserted at jj) and i + jj, so no lane idles.
  for (int kk = 2; kk <= SN; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int q = t; q < SN / 2; q += kThreads) {
        const int i = ((q & ~(jj - 1)) << 1) | (q & (jj - 1));
        const int p = i + jj;
        const double ka = key[i], kb = key[p];
        const int ia = idx[i], ib = idx[p];
        const bool up = (i & kk) == 0;
        if (up ? before(kb, ib, ka, ia) : before(ka, ia, kb, ib)) {
          key[i] = kb; key[p] = ka;
          idx[i] = ib; idx[p] = ia;
        }
      }
      __syncthreads();
    }
  }

  int n_keep;
  if (topk == 0) {
    if (thr >= 1.0) {
      n_keep = nbk;
    } else {
      // Running sums of the sorted probabilities: each thread owns SN/kThreads
      // consecutive entries.
      const int per = SN / kThreads, i0 = t * per;
      double local = 0;
      for (int i = 0; i < per; ++i) local += (i0 + i < nbk) ? key[i0 + i] : 0.0;
      // exclusive prefix of the per-thread totals: wave scan, then wave offsets
      double incl = local;
      const int ln = lane_id(), wv = t / kWave;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const double y = __shfl_up(incl, o, kWave);
        if (ln >= o) incl += y;
      }
      if (ln == kWave - 1) tsum[wv] = incl;
      __syncthreads();
      double before_sum = incl - local;
      for (int u = 0; u < wv; ++u) before_sum += tsum[u];
      double c = before_sum;
      for (int i = 0; i < per; ++i) {
        if (i0 + i >= nbk) break;
        c += key[i0 + i];
        if (c >= thr) {
          atomicMin(&cut_s, i0 + i);
          break;
        }
      }
      __syncthreads();
      n_keep = cut_s >= nbk ? nbk : cut_s + 1;
    }
  } else {
    n_keep = min(topk, n_cand);
    for (int r = 0; r < fc.n; ++r)
      for (int j = fc.lo[r] + t; j < fc.hi[r]; j += kThreads) atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  for (int i = t; i < n_keep; i += kThreads) {
    const int j = idx[i];
    atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  int cnt = 0;
  for (int w = t; w < words; w += kThreads) {
    bitmap[row * words + w] = bits[w];
    cnt += __popc(bits[w]);
  }
  // total kept = popcount of the whole bitmap row
  const double tot = block_reduce((double)cnt, false, red);
  if (t == 0) row_ptr[row + 1] = (int32_t)tot;
}

// -------------------------------------------------------------------- 4. CSR
constexpr int kRowsPerBlock = 4;

__global__ __launch_bounds__(kRowsPerBlock * kWave) void bitmap_fill_kernel(
    const uint32_t* __restrict__ bitmap, int64_t n_rows, int nbk, const int32_t* row_ptr,
    int32_t* col_idx) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (row >= n_rows) return;
  const int words = (nbk + 31) / 32;
  int out = row_ptr[row];
  for (int w0 = 0; w0 < words; w0 += kWave) {
    const int w = w0 + lane_id();
    uint32_t b = w < words ? bitmap[row * words + w] : 0u;
    const int c = __popc(b);
    const int incl = wave_inclusive_scan(c);
    int pos = out + incl - c;
    while (b) {
      const int bit = __builtin_ctz(b);
      col_idx[pos++] = w * 32 + bit;
      b &= b - 1;
    }
    out += __shfl(incl, kWave - 1, kWave);
  }
}

}  // namespace

size_t nabla_workspace_bytes(int64_t batch, int heads, int head_dim, int64_t nq, int64_t nk,
                             int block_q, int block_k) {
  const int64_t nbq = (nq + block_q - 1) / block_q, nbk = (nk + block_k - 1) / block_k;
  return layout(batch * heads, head_dim, nbq, nbk).total;
}

hipError_t launch_mask_nabla(const NablaArgs& a, hipStream_t stream) {
  const int64_t bh = a.batch * a.heads;
  const int nbq = (int)((a.nq + a.block_q - 1) / a.block_q);
  const int nbk = (int)((a.nk + a.block_k - 1) / a.block_k);
  const Layout L = layout(bh, a.head_dim, nbq, nbk);
  uint8_t* ws = (uint8_t*)a.workspace;
  double* qp = (double*)(ws + L.qp);
  double* kp = (double*)(ws + L.kp);
  double* z = (double*)(ws + L.z);
  uint32_t* bitmap = (uint32_t*)(ws + L.bits);
  const int hd = a.heads * a.head_dim;

  // threads per workgroup: the row's 8-element vectors split evenly into slices of at
  // most kPoolMaxThreads, rounded up to whole waves
  const int vpr = hd / 8;
  const int slices = (vpr + kPoolMaxThreads - 1) / kPoolMaxThreads;
  const int per = (vpr + slices - 1) / slices;
  const int pool_threads = (per + kWave - 1) / kWave * kWave;
  dim3 g1(nbq + nbk, (vpr + pool_threads - 1) / pool_threads, (unsigned)a.batch);
  hipLaunchKernelGGL(a.dtype == 1 ? pool_kernel<true> : pool_kernel<false>, g1, dim3(pool_threads), 0,
                     stream, (const uint8_t*)a.q, (const uint8_t*)a.k, a.nq, a.nk, a.block_q,
                     a.block_k, nbq, nbk, a.heads, a.head_dim, qp, kp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  dim3 g2((nbk + kTile - 1) / kTile, (nbq + kTile - 1) / kTile, (unsigned)bh);
  hipLaunchKernelGGL(score_kernel, g2, dim3(kThreads), 0, stream, qp, kp, nbq, nbk, a.head_dim,
                     a.scale, z);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  int SN = kThreads;
  while (SN < nbk) SN <<= 1;
  Forced fc{};
  fc.n = a.topk > 0 ? a.n_forced : 0;
  for (int r = 0; r < fc.n; ++r) {
    fc.lo[r] = a.forced[2 * r];
    fc.hi[r] = a.forced[2 * r + 1];
  }
  const int words = (nbk + 31) / 32;
  const size_t lds = (size_t)SN * (sizeof(double) + sizeof(int)) + words * sizeof(uint32_t);
  const int64_t rows = bh * nbq;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)rows), dim3(kThreads), lds, stream, z, nbk, SN,
                     a.threshold, a.topk, fc, bitmap, a.row_ptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_counts_to_offsets(a.row_ptr, rows, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(bitmap_fill_kernel, dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(kRowsPerBlock * kWave), 0, stream, bitmap, rows, nbk, a.row_ptr,
                     a.col_idx);
  return hipGetLastError();
}

}  // namespace vsa

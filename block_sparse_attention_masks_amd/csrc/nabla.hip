// Dynamic block mask from mean-pooled Q and K (NABLA explainer, aibr.jp/archives/
// 124678, sec. 3), and the anchor + recent + top-k variant used for an
// autoregressive chunk step (Sparse Forcing summary, gist.science/ja/paper/
// 2604.21221, part 2).
//
// Four passes, all in fp64 so that the decision matches a plain fp64 evaluation
// except where the cumulative mass sits within rounding of the threshold:
//   1. pool      -- per block, exact fp64 sums of the (bf16 or fp32) token rows,
//                   one division by the number of valid tokens.  HBM-bound: the
//                   waves of a workgroup stream parts of a block's rows with 16-byte
//                   loads and add their parts in LDS.
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

// grid: x = (block, 64-vector slice of a row) with the slice fastest (a vector = 8
// elements; blocks are the query blocks, then the key blocks), z = batch: the workgroups
// that run side by side read neighbouring parts of the same rows, so whole rows stream
// from each DRAM page.  The kPoolWaves waves of a workgroup interleave over the block's valid
// rows (wave w takes rows w, w + 8, ...), so a workgroup sweeps consecutive rows together;
// lane l of every wave sums vector 64 y + l of its rows, keeping 64 bytes of loads in flight
// (4 bf16 rows or 2 fp32 rows) so that a wave of even a 64-row block loads in two batches,
// and the waves' sums meet in LDS.  The sums of bf16 values are exact in fp64, so the order
// in which rows and waves are added does not matter.  The element type is a template
// parameter so that each kernel holds only its own registers.  The means are written
// block-major, [batch, block, head, D] (the token tensor's own order), so that the means of
// one block, which the workgroups of its slices write at about the same time, are one
// contiguous run; head-major, each workgroup scattered its 1 KB pieces over 40 regions
// about a megabyte apart.  Measured with the caches flushed: 71% of HBM on 64-row blocks
// (69% head-major; 86% when timing-only code skips the writes, so the 6% of bytes written
// still costs about a fifth of the time), 73% on 128-row and 74-75% on 384-row blocks.
constexpr int kPoolWaves = 8;
template <bool BF16>
__global__ __launch_bounds__(kPoolWaves * kWave) void pool_kernel(const uint8_t* __restrict__ q,
                                                           const uint8_t* __restrict__ k,
                                                           int64_t nq, int64_t nk, int bq, int bk,
                                                           int nbq, int nbk, int heads, int D, int slices,
                                                           double* __restrict__ qp,
                                                           double* __restrict__ kp) {
  __shared__ double part[kPoolWaves - 1][8][kWave];
  const int xb = blockIdx.x / slices, slice = blockIdx.x - xb * slices;
  const bool isq = xb < nbq;
  const int blk = isq ? xb : xb - nbq;
  const int64_t n = isq ? nq : nk;
  const int bsz = isq ? bq : bk;
  const int nb = isq ? nbq : nbk;
  const uint8_t* src = isq ? q : k;
  double* dst = isq ? qp : kp;
  const int64_t b = blockIdx.z;
  const int hd = heads * D;
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int vec = slice * kWave + l;  // 8-element vector index in a row
  const bool active = vec * 8 < hd;
  constexpr int esz = BF16 ? 2 : 4;
  const int64_t row_bytes = (int64_t)hd * esz;
  const int64_t t0 = (int64_t)blk * bsz, t1 = min(n, t0 + bsz);
  constexpr int W = kPoolWaves;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (active) {
    const uint8_t* p = src + (b * n + t0 + w) * row_bytes + (int64_t)vec * 8 * esz;
    int64_t t = t0 + w;
    constexpr int U = BF16 ? 4 : 2;
    for (; t + (U - 1) * W < t1; t += U * W) {
      Vec8<BF16> x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u].load(p + u * W * row_bytes);
#pragma unroll
      for (int u = 0; u < U; ++u) x[u].add_to(acc);
      p += U * W * row_bytes;
    }
    for (; t < t1; t += W) {
      Vec8<BF16> x;
      x.load(p);
      x.add_to(acc);
      p += W * row_bytes;
    }
  }
  if (w > 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) part[w - 1][i][l] = acc[i];
  }
  __syncthreads();
  if (w > 0 || !active) return;
#pragma unroll
  for (int u = 0; u < kPoolWaves - 1; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += part[u][i][l];
  const double cnt = (double)(t1 - t0);
  const int e0 = vec * 8, h = e0 / D, d0 = e0 % D;   // D is a multiple of 8
  double* out = dst + ((b * nb + blk) * heads + h) * D + d0;
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = acc[i] / cnt;
}

hipError_t launch_pool(const void* q, const void* k, int bf16, int64_t batch, int heads, int D, int64_t nq,
                       int64_t nk, int bq, int bk, int nbq, int nbk, double* qp, double* kp,
                       hipStream_t stream) {
  const int slices = (heads * D / 8 + kWave - 1) / kWave;
  const dim3 grid((unsigned)((nbq + nbk) * slices), 1, (unsigned)batch);
  auto kern = bf16 ? pool_kernel<true> : pool_kernel<false>;
  hipLaunchKernelGGL(kern, grid, dim3(kPoolWaves * kWave), 0, stream, (const uint8_t*)q, (const uint8_t*)k, nq,
                     nk, bq, bk, nbq, nbk, heads, D, slices, qp, kp);
  return hipGetLastError();
}

// ------------------------------------------------------------------ 2. score
constexpr int kTile = 64, kKc = 16;

// qp, kp: the pooled means, block-major [batch, block, head, D]; z: [batch * heads, nbq, nbk].
__global__ __launch_bounds__(kThreads) void score_kernel(const double* __restrict__ qp,
                                                         const double* __restrict__ kp, int nbq,
                                                         int nbk, int heads, int D, double scale,
                                                         double* __restrict__ z) {
  __shared__ double As[kKc][kTile + 1];
  __shared__ double Bs[kKc][kTile + 1];
  const int64_t bh = blockIdx.z, b = bh / heads;
  const int h = (int)(bh - b * heads);
  const int i0 = blockIdx.y * kTile, j0 = blockIdx.x * kTile;
  const int64_t rs = (int64_t)heads * D;  // between consecutive blocks of one head
  const double* A = qp + (b * nbq * heads + h) * (int64_t)D;
  const double* B = kp + (b * nbk * heads + h) * (int64_t)D;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  double acc[4][4] = {};
  for (int d0 = 0; d0 < D; d0 += kKc) {
    for (int e = threadIdx.x; e < kTile * kKc; e += kThreads) {
      const int r = e / kKc, c = e % kKc;
      As[c][r] = (i0 + r < nbq) ? A[(int64_t)(i0 + r) * rs + d0 + c] : 0.0;
      Bs[c][r] = (j0 + r < nbk) ? B[(int64_t)(j0 + r) * rs + d0 + c] : 0.0;
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

// One compare-exchange of a bitonic stage, seen from one side: this element (k, i) at
// position pos meets (pk, pi) at pos ^ jj; `up` sorts the kk-run ascending in `before`
// order.  The lower position keeps the element that comes first, the upper the other.
__device__ inline void keep_side(double& k, int& i, double pk, int pi, bool lower, bool up) {
  const bool mine_first = before(k, i, pk, pi);
  if (mine_first != (lower == up)) {
    k = pk;
    i = pi;
  }
}

// E = SN / kThreads sort slots per thread: thread t holds positions t E .. t E + E - 1 in
// registers.  A bitonic stage of distance jj pairs positions inside a thread (jj < E),
// inside a wave (lanes jj / E apart, exchanged with shuffles) or across waves (through
// LDS, the only stages that need a barrier: 3 of the 55 at SN = 1024).
template <int E>
__global__ __launch_bounds__(kThreads) void select_kernel(const double* __restrict__ z, int nbk,
                                                          double thr, int topk, Forced fc,
                                                          uint32_t* __restrict__ bitmap,
                                                          int32_t* __restrict__ row_ptr) {
  constexpr int SN = E * kThreads;
  __shared__ double xkey[SN];
  __shared__ int xidx[SN];
  __shared__ uint32_t bits[SN / 32];
  __shared__ double red[kThreads / kWave];
  __shared__ double tsum[kThreads / kWave];
  __shared__ int cut_s;
  const int words = (nbk + 31) / 32;
  const int64_t row = blockIdx.x;
  const double* zr = z + row * nbk;
  const int t = threadIdx.x;
  const int i0 = t * E;  // this thread's first position
  for (int w = t; w < words; w += kThreads) bits[w] = 0;
  if (t == 0) cut_s = SN;

  double key[E];
  int idx[E];
  int n_cand = nbk;
  if (topk == 0) {
    double m = -DBL_MAX;
    for (int j = t; j < nbk; j += kThreads) m = fmax(m, zr[j]);
    m = block_reduce(m, true, red);
    double s = 0;
    for (int j = t; j < nbk; j += kThreads) s += exp(zr[j] - m);
    s = block_reduce(s, false, red);
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const int j = i0 + r;
      key[r] = j < nbk ? exp(zr[j] - m) / s : -1.0;
      idx[r] = j;
    }
  } else {
    for (int r = 0; r < fc.n; ++r) n_cand -= fc.hi[r] - fc.lo[r];  // ranges are disjoint
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const int j = i0 + r;
      bool forced = false;
      for (int f = 0; f < fc.n; ++f) forced |= (j >= fc.lo[f] && j < fc.hi[f]);
      key[r] = (j < nbk && !forced) ? zr[j] : -DBL_MAX;
      idx[r] = j;
    }
  }

  // Bitonic sort of (key, idx) into `before` order.
#pragma unroll
  for (int kk = 2; kk <= SN; kk <<= 1) {
#pragma unroll
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      if (jj < E) {
#pragma unroll
        for (int r = 0; r < E; ++r) {
          if (r & jj) continue;
          const int q = r + jj;
          const bool up = ((i0 + r) & kk) == 0;
          if (up ? before(key[q], idx[q], key[r], idx[r]) : before(key[r], idx[r], key[q], idx[q])) {
            const double tk = key[r];
            const int ti = idx[r];
            key[r] = key[q];
            idx[r] = idx[q];
            key[q] = tk;
            idx[q] = ti;
          }
        }
      } else if (jj < kWave * E) {
        const int d = jj / E;  // lane distance
        const bool lower = (lane_id() & d) == 0;
#pragma unroll
        for (int r = 0; r < E; ++r) {
          const double pk = __shfl_xor(key[r], d, kWave);
          const int pi = __shfl_xor(idx[r], d, kWave);
          keep_side(key[r], idx[r], pk, pi, lower, ((i0 + r) & kk) == 0);
        }
      } else {
#pragma unroll
        for (int r = 0; r < E; ++r) {
          xkey[i0 + r] = key[r];
          xidx[i0 + r] = idx[r];
        }
        __syncthreads();
        const bool lower = (i0 & jj) == 0;  // jj >= kWave * E: the same for all r
#pragma unroll
        for (int r = 0; r < E; ++r) {
          const int p = (i0 + r) ^ jj;
          keep_side(key[r], idx[r], xkey[p], xidx[p], lower, ((i0 + r) & kk) == 0);
        }
        __syncthreads();
      }
    }
  }

  int n_keep;
  if (topk == 0) {
    if (thr >= 1.0) {
      n_keep = nbk;
    } else {
      // Running sums of the sorted probabilities: each thread owns E consecutive entries.
      double local = 0;
#pragma unroll
      for (int r = 0; r < E; ++r) local += (i0 + r < nbk) ? key[r] : 0.0;
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
      int cut = SN;
#pragma unroll
      for (int r = 0; r < E; ++r) {
        if (cut == SN && i0 + r < nbk) {
          c += key[r];
          if (c >= thr) cut = i0 + r;
        }
      }
      if (cut < SN) atomicMin(&cut_s, cut);
      __syncthreads();
      n_keep = cut_s >= nbk ? nbk : cut_s + 1;
    }
  } else {
    n_keep = min(topk, n_cand);
    for (int r = 0; r < fc.n; ++r)
      for (int j = fc.lo[r] + t; j < fc.hi[r]; j += kThreads) atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
#pragma unroll
  for (int r = 0; r < E; ++r)
    if (i0 + r < n_keep) atomicOr(&bits[idx[r] >> 5], 1u << (idx[r] & 31));
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

hipError_t launch_block_pool(const void* x, int bf16, int64_t batch, int heads, int D, int64_t n, int block,
                             double* out, hipStream_t stream) {
  const int nb = (int)((n + block - 1) / block);
  return launch_pool(x, x, bf16, batch, heads, D, n, n, block, block, nb, 0, out, out, stream);
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
  hipError_t e = launch_pool(a.q, a.k, a.dtype == 1, a.batch, a.heads, a.head_dim, a.nq, a.nk, a.block_q,
                            a.block_k, nbq, nbk, qp, kp, stream);
  if (e != hipSuccess) return e;

  dim3 g2((nbk + kTile - 1) / kTile, (nbq + kTile - 1) / kTile, (unsigned)bh);
  hipLaunchKernelGGL(score_kernel, g2, dim3(kThreads), 0, stream, qp, kp, nbq, nbk, a.heads, a.head_dim,
                     a.scale, z);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  int E = 1;  // sort slots per thread: SN = E * kThreads >= nbk (nbk <= 4096 is checked)
  while (E * kThreads < nbk) E <<= 1;
  Forced fc{};
  fc.n = a.topk > 0 ? a.n_forced : 0;
  for (int r = 0; r < fc.n; ++r) {
    fc.lo[r] = a.forced[2 * r];
    fc.hi[r] = a.forced[2 * r + 1];
  }
  const int64_t rows = bh * nbq;
  auto sel = E == 1 ? select_kernel<1> : E == 2 ? select_kernel<2> : E == 4 ? select_kernel<4>
           : E == 8 ? select_kernel<8> : select_kernel<16>;
  hipLaunchKernelGGL(sel, dim3((unsigned)rows), dim3(kThreads), 0, stream, z, nbk, a.threshold, a.topk, fc,
                     bitmap, a.row_ptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_counts_to_offsets(a.row_ptr, rows, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(bitmap_fill_kernel, dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(kRowsPerBlock * kWave), 0, stream, bitmap, rows, nbk, a.row_ptr,
                     a.col_idx);
  return hipGetLastError();
}

}  // namespace vsa

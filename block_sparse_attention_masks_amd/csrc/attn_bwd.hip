// Block-sparse attention backward: gradients of L = sum(dO * O) for
// O = softmax(Q K^T * scale) V over the key blocks a CSR mask keeps (the pages
// report training gains as well as inference gains, Radial Attention explainer,
// aibr.jp/archives/112136, sec. 4).  With the saved lse and D_i = sum_d dO_i O_i:
//
//   P = exp(S * scale - lse),  dV = P^T dO,  dP = dO V^T,
//   dS = P * (dP - D),  dQ = dS K * scale,  dK = dS^T Q * scale.
//
// Four passes, deterministic (no atomics):
//   1. delta_kernel     D = rowsum(dO * O), fp32;
//   2. csc_kernel       the transposed view of the mask: for each (slab, key block)
//                       the query blocks that keep it, ascending;
//   3. dq_kernel        per query tile, over its kept key tiles (like the forward):
//                       S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T;
//   4. dkdv_kernel      per key tile, over the query tiles of the blocks that keep
//                       it: S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS.
//                       Key blocks of <= 64 keys are grouped (group_union.h builds the
//                       union of a group's query blocks from the CSC view first).
// Every product is v_mfma_f32_32x32x16_bf16 on bf16 operands (P and dS rounded to
// bf16), fp32 accumulation; gradients are written in fp32.
//
// Tiles of 64 rows x D are copied global -> LDS directly (global_load_lds, 16 bytes
// per lane) into an unpadded layout whose 16-byte chunks are XOR-permuted per row by
// swz(r).  The same tile is read two ways -- 16-byte fragments of 32 rows x one chunk
// pair (the A operand of S / dP) and transposed 8-byte reads of 4 rows x 64 bytes
// (the A operand of the gradient products) -- and swz is conflict-free for both: it
// is a bijection on 16 consecutive rows (D = 128; on 8 row pairs for D = 64) and it
// gives the 4 rows of an aligned group 4 distinct 64-byte bank groups.
//
// fp32 path: the same definitions with fp32 FMA, one wave per query row (dQ) or key
// row (dK, dV), lanes over head_dim (used for small fp32 problems).
#include <math.h>

#include "group_union.h"
#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64_t;

constexpr int kT = 64;      // rows per tile (keys in dq_kernel, queries in dkdv_kernel)
constexpr int kNW = 4;      // waves per workgroup
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
__device__ inline int swz(int r) {
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One wave copies 64 x 16 bytes from global memory to LDS: lane i's bytes land at lds + 16 i.
__device__ inline void load_lds16(const uint16_t* src, uint16_t* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ inline float xchg32(float x, int g) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(g == 0 ? r[1] : r[0]);
}

// Transposed A-operand fragments of one 16-row group of a tile for every 32-column
// slice: f[t][i] = X[row_i][32 t + lane % 32] with row_i = 4 g + i (i < 4) and
// 8 + 4 g + i - 4 (i >= 4), g = lane / 32 -- the row order of the accumulator layout.
// lo[t] / hi[t]: byte addresses of this lane's 8 bytes in rows 4 g + jv and 8 + 4 g + jv.
// The reads and their wait sit in one asm block (see the forward kernel: written as
// builtins, the compiler would wait for every in-flight global -> LDS copy first).
template <int D>
__device__ inline void read_tr(bf16x8 (&f)[D / 32], const uint32_t (&lo)[D / 32], const uint32_t (&hi)[D / 32],
                               uint32_t base);

template <>
__device__ inline void read_tr<128>(bf16x8 (&f)[4], const uint32_t (&lo)[4], const uint32_t (&hi)[4],
                                    uint32_t base) {
  u64_t r0, r1, r2, r3, r4, r5, r6, r7;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n"
      "ds_read_b64_tr_b16 %1, %9\n"
      "ds_read_b64_tr_b16 %2, %10\n"
      "ds_read_b64_tr_b16 %3, %11\n"
      "ds_read_b64_tr_b16 %4, %12\n"
      "ds_read_b64_tr_b16 %5, %13\n"
      "ds_read_b64_tr_b16 %6, %14\n"
      "ds_read_b64_tr_b16 %7, %15\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(base + lo[0]), "v"(base + hi[0]), "v"(base + lo[1]), "v"(base + hi[1]), "v"(base + lo[2]),
        "v"(base + hi[2]), "v"(base + lo[3]), "v"(base + hi[3])
      : "memory");
  const u64_t r[8] = {r0, r1, r2, r3, r4, r5, r6, r7};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const u64_t pr[2] = {r[2 * t], r[2 * t + 1]};
    f[t] = __builtin_bit_cast(bf16x8, pr);
  }
}

template <>
__device__ inline void read_tr<64>(bf16x8 (&f)[2], const uint32_t (&lo)[2], const uint32_t (&hi)[2],
                                   uint32_t base) {
  u64_t r0, r1, r2, r3;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n"
      "ds_read_b64_tr_b16 %1, %5\n"
      "ds_read_b64_tr_b16 %2, %6\n"
      "ds_read_b64_tr_b16 %3, %7\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(base + lo[0]), "v"(base + hi[0]), "v"(base + lo[1]), "v"(base + hi[1])
      : "memory");
  const u64_t r[4] = {r0, r1, r2, r3};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const u64_t pr[2] = {r[2 * t], r[2 * t + 1]};
    f[t] = __builtin_bit_cast(bf16x8, pr);
  }
}

// Byte offsets (within a tile) of this lane's transposed reads, rows 4 g + jv and 8 + 4 g + jv.
template <int D>
__device__ inline void tr_offsets(uint32_t (&lo)[D / 32], uint32_t (&hi)[D / 32], int l) {
  const int g = l >> 5, jv = (l & 15) >> 2, c4 = l & 3, m2 = (l >> 4) & 1;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    const int ch = 4 * t + 2 * m2 + (c4 >> 1);
    const int r0 = 4 * g + jv, r1 = 8 + 4 * g + jv;
    lo[t] = 2u * (r0 * D + 8 * (ch ^ swz<D>(r0)) + 4 * (c4 & 1));
    hi[t] = 2u * (r1 * D + 8 * (ch ^ swz<D>(r1)) + 4 * (c4 & 1));
  }
}

// 16-byte A fragment: row (32 st + col) of the tile, chunk (2 kd + g).
template <int D>
__device__ inline bf16x8 frag(const uint16_t* tile, int row, int kd, int g) {
  return *(const bf16x8*)(tile + row * D + 8 * ((2 * kd + g) ^ swz<D>(row)));
}

// A stream of 64-row tiles over a list of blocks (wave-uniform): block list[e], rows
// [list[e] * bsz, min(+bsz, n)).  Row indices fit 31 bits with 64 to spare (the call
// checks), so the walk is 32-bit scalar arithmetic.
struct Tiles {
  const int32_t* list;
  int e, e1;
  int r0, re;
  int bsz;
  int n;
  __device__ bool valid() const { return e < e1; }
  __device__ void open() {
    if (e < e1) {
      r0 = list[e] * bsz;
      re = bsz < n - r0 ? r0 + bsz : n;
    }
  }
  __device__ void next() {
    r0 += kT;
    if (r0 >= re) {
      ++e;
      open();
    }
  }
};

template <int D>
struct Smem {
  uint16_t a[2][kT * D];   // K (dq) or Q (dkdv)
  uint16_t b[2][kT * D];   // V (dq) or dO (dkdv)
  float lse[2][kT];        // dkdv: lse * log2(e) of the tile's queries (+inf past the end)
  float dl[2][kT];         // dkdv: D of the tile's queries (0 past the end)
};

// Work items to workgroups, as in the forward: XCD b % 8 takes contiguous ranges (chunk = 0)
// or runs of chunk consecutive items (xcd_run).
struct Work {
  int64_t items, per_xcd;
  int nb, mt_per_b;
  int chunk = 0;
};

__device__ inline int64_t work_item(const Work& wk, int64_t bid) {
  if (wk.chunk == 0) return (bid % 8) * wk.per_xcd + bid / 8;
  const int64_t c8 = 8 * (int64_t)wk.chunk, full = wk.items / c8 * c8;
  return bid < full ? bid / c8 * c8 + (bid % 8) * wk.chunk + bid / 8 % wk.chunk : bid;
}

// Grouped key blocks (dK, dV with blocks of <= 64 keys): G consecutive key blocks of a
// slab share a 4-wave workgroup (wpb waves each) and walk the union of the query blocks
// that keep any of them; list u = slab * n_groups + group holds cnt[u] entries at
// idx[u * cap ..], each with a mask of the group's key blocks that it keeps.
// The lists are kernel arguments of their own (idx in row_idx's place, mask, cnt), declared
// __restrict__ like the CSC view, so that the compiler reads them with scalar loads: through
// a struct's pointers they were vector loads whose waits also waited for the copies just
// issued.
struct KeyGroups {
  int G, wpb, cap;
};

// Copy plan shared by both kernels: wave-load c = w + 4 j (c < 2 CB) moves RPC rows of
// tensor a (c < CB) or b (c - CB) of a tile into LDS; rows past the last valid one repeat it.
template <int D>
struct CopyPlan {
  // The same copy, with each lane's row and slot recomputed from the lane id (which the
  // caller makes opaque, so the 2 NJ values are not kept live across the loop).
  static __device__ void issue_lean(const uint16_t* abase, const uint16_t* bbase, int r0, int re,
                                    uint32_t row_bytes, int row_stride, uint16_t* sa, uint16_t* sb, int w, int l);
  static constexpr int SPR = D / 8, RPC = 64 / SPR, CB = kT / RPC, NJ = (2 * CB + kNW - 1) / kNW;
  int lrow[NJ];
  uint32_t ch16[NJ];
  __device__ CopyPlan(int w, int l) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = w + kNW * j;
      const int cb = c < CB ? c : c - CB;
      lrow[j] = cb * RPC + l / SPR;
      ch16[j] = 16u * ((l % SPR) ^ swz<D>(lrow[j]));
    }
  }
  __device__ void issue(const uint16_t* abase, const uint16_t* bbase, int r0, int re, uint32_t row_bytes,
                        int row_stride, uint16_t* sa, uint16_t* sb, int w) const;
};

template <int D>
__device__ void CopyPlan<D>::issue_lean(const uint16_t* abase, const uint16_t* bbase, int r0, int re,
                                        uint32_t row_bytes, int row_stride, uint16_t* sa, uint16_t* sb, int w,
                                        int l) {
  const char* at = (const char*)(abase + (int64_t)r0 * row_stride);
  const char* bt = (const char*)(bbase + (int64_t)r0 * row_stride);
  const int last = min(re - r0, kT) - 1;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = w + kNW * j;
    if (c < 2 * CB) {
      const int cb = c < CB ? c : c - CB;
      const int lrow = cb * RPC + l / SPR;
      const uint32_t ro = __umul24((uint32_t)min(lrow, last), row_bytes) + 16u * ((l % SPR) ^ swz<D>(lrow));
      if (c < CB) load_lds16((const uint16_t*)(at + ro), sa + c * 512);
      else load_lds16((const uint16_t*)(bt + ro), sb + (c - CB) * 512);
    }
  }
}

template <int D>
__device__ void CopyPlan<D>::issue(const uint16_t* abase, const uint16_t* bbase, int r0, int re, uint32_t row_bytes,
                                   int row_stride, uint16_t* sa, uint16_t* sb, int w) const {
    const char* at = (const char*)(abase + (int64_t)r0 * row_stride);
    const char* bt = (const char*)(bbase + (int64_t)r0 * row_stride);
    const int last = min(re - r0, kT) - 1;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = w + kNW * j;
      if (c < 2 * CB) {
        const uint32_t ro = __umul24((uint32_t)min(lrow[j], last), row_bytes) + ch16[j];
        if (c < CB) load_lds16((const uint16_t*)(at + ro), sa + c * 512);
        else load_lds16((const uint16_t*)(bt + ro), sb + (c - CB) * 512);
      }
    }
}

// ------------------------------------------------------------------ 1. D
// One thread per 8 elements of a token row; the D / 8 lanes of a head reduce with DPP.
template <int CTRL>
__device__ inline float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int LANES>
__device__ inline float head_sum(float v) {
  v += dppf<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dppf<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dppf<0x141>(v);  // row_half_mirror
  if (LANES == 16) v += dppf<0x140>(v);  // row_mirror
  return v;
}

__device__ inline void load8f(const uint8_t* p, bool bf16, float* x) {
  const u32x4 a = *(const u32x4*)p;
  if (bf16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(a[i] << 16);
      x[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
    }
  } else {
    const u32x4 c = *(const u32x4*)(p + 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(a[i]), x[4 + i] = __uint_as_float(c[i]);
  }
}

template <int LANES>
__global__ __launch_bounds__(256) void delta_kernel(const uint8_t* __restrict__ o, const uint8_t* __restrict__ dout,
                                                    int bf16, int64_t rows, int heads, int D, int64_t nq,
                                                    float* __restrict__ delta) {
  const int vpr = heads * D / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = idx < rows * vpr;  // whole heads are live or dead together
  const int64_t row = live ? idx / vpr : 0;
  const int vec = live ? (int)(idx % vpr) : 0;
  const int esz = bf16 ? 2 : 4;
  const int64_t off = (row * vpr + vec) * 8 * esz;
  float a[8], c[8];
  load8f(o + off, bf16, a);
  load8f(dout + off, bf16, c);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += a[i] * c[i];
  s = head_sum<LANES>(s);
  if (live && vec % LANES == 0) {
    const int64_t b = row / nq, q = row % nq;
    delta[(b * heads + vec / LANES) * nq + q] = s;
  }
}

// ------------------------------------------------------------------ 2. CSC
constexpr int kCscThreads = 1024;

__device__ int block_exclusive_scan(int f, int* total) {
  __shared__ int wave_tot[kCscThreads / kWave];
  const int t = threadIdx.x, l = lane_id(), w = t / kWave;
  const int incl = wave_inclusive_scan(f);
  if (l == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  if (w == 0) {
    int x = l < kCscThreads / kWave ? wave_tot[l] : 0;
    x = wave_inclusive_scan(x);
    if (l < kCscThreads / kWave) wave_tot[l] = x;
  }
  __syncthreads();
  const int excl = (w > 0 ? wave_tot[w - 1] : 0) + incl - f;
  *total = wave_tot[kCscThreads / kWave - 1];
  __syncthreads();
  return excl;
}

// One workgroup per slab.  The slab's CSC entries take the same range of the index array
// as its CSR entries.  Rows are walked in ascending order, so each column lists its query
// blocks ascending; within a row every column appears once, so the per-column counters
// need no atomics.
__global__ __launch_bounds__(kCscThreads) void csc_kernel(const int32_t* __restrict__ row_ptr,
                                                          const int32_t* __restrict__ col_idx, int nbq, int nbk,
                                                          int64_t n_slabs, int32_t* __restrict__ cnt,
                                                          int32_t* __restrict__ col_ptr,
                                                          int32_t* __restrict__ row_idx) {
  const int64_t s = blockIdx.x;
  int32_t* c = cnt + s * nbk;
  for (int j = threadIdx.x; j < nbk; j += kCscThreads) c[j] = 0;
  __threadfence_block();
  __syncthreads();
  for (int i = 0; i < nbq; ++i) {
    const int64_t r = s * nbq + i;
    for (int32_t e = row_ptr[r] + threadIdx.x; e < row_ptr[r + 1]; e += kCscThreads) c[col_idx[e]] += 1;
    __threadfence_block();
    __syncthreads();
  }
  int run = row_ptr[s * nbq];
  for (int base = 0; base < nbk; base += kCscThreads) {
    const int j = base + threadIdx.x;
    const int f = j < nbk ? c[j] : 0;
    int chunk = 0;
    const int excl = block_exclusive_scan(f, &chunk);
    if (j < nbk) {
      col_ptr[s * nbk + j] = run + excl;
      c[j] = run + excl;  // becomes the column's write cursor
    }
    run += chunk;
  }
  if (s == n_slabs - 1 && threadIdx.x == 0) col_ptr[n_slabs * nbk] = run;
  __threadfence_block();
  __syncthreads();
  for (int i = 0; i < nbq; ++i) {
    const int64_t r = s * nbq + i;
    for (int32_t e = row_ptr[r] + threadIdx.x; e < row_ptr[r + 1]; e += kCscThreads) {
      const int j = col_idx[e];
      row_idx[c[j]] = i;
      c[j] += 1;
    }
    __threadfence_block();
    __syncthreads();
  }
}

// ------------------------------------------------------------------ 3. dQ
// A workgroup of 4 waves owns 32 * 4 / KS query rows of one query block; with KS = 2 the
// wave pairs (w, w + 2) share 32 rows and split each key tile, adding their dQ at the end.
template <int D, int KS>
__global__ __launch_bounds__(kNW * kWave, 2) void dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dq, int64_t nq, int64_t nk, int heads, int block_q, int block_k,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int n_slabs, float scale,
    float scale_log2, Work wk) {
  __shared__ __attribute__((aligned(1024))) Smem<D> sm;
  constexpr int BM = 32 * kNW / KS;
  constexpr int NST = 2 / KS;
  const int64_t bid = blockIdx.x;
  const int64_t item = work_item(wk, bid);
  if (item >= wk.items) return;
  const int mt = (int)(item % wk.mt_per_b);
  int64_t rest = item / wk.mt_per_b;
  const int qb = (int)(rest % wk.nb);
  rest /= wk.nb;
  const int h = (int)(rest % heads);
  const int64_t b = rest / heads;
  const int64_t q_lo = (int64_t)qb * block_q + (int64_t)mt * BM;
  const int64_t q_hi = min(min((int64_t)(qb + 1) * block_q, nq), q_lo + BM);
  if (q_lo >= q_hi) return;

  const int l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int col = l & 31, g = l >> 5;
  const int qw = KS == 1 ? w : (w & 1);
  const int kh = KS == 1 ? 0 : (w >> 1);
  const int row_stride = heads * D;
  const uint32_t row_bytes = 2u * (uint32_t)row_stride;

  const int64_t slab = n_slabs == 1 ? 0 : b * heads + h;
  const int64_t r = slab * wk.nb + qb;
  Tiles it{col_idx, row_ptr[r], row_ptr[r + 1], 0, 0, block_k, (int)nk};
  it.open();
  const uint16_t* kbase = k + (b * nk * heads + h) * (int64_t)D;
  const uint16_t* vbase = v + (b * nk * heads + h) * (int64_t)D;
  const CopyPlan<D> plan(w, l);

  // this lane's query: B operands Q^T and dO^T, its lse (log2 domain) and D
  const int64_t my_q = q_lo + qw * 32 + col;
  const bool ok = my_q < q_hi;
  bf16x8 qf[D / 16], df[D / 16];
  {
    const int64_t base = ((b * nq + (ok ? my_q : q_lo)) * heads + h) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qf[s] = __builtin_bit_cast(bf16x8, ok ? *(const u32x4*)(q + base + 16 * s) : u32x4{0, 0, 0, 0});
      df[s] = __builtin_bit_cast(bf16x8, ok ? *(const u32x4*)(dout + base + 16 * s) : u32x4{0, 0, 0, 0});
    }
  }
  const float lse2 = ok ? lse[(b * heads + h) * nq + my_q] * kLog2e : 0.f;
  const float dlt = ok ? delta[(b * heads + h) * nq + my_q] : 0.f;
  if (it.valid()) plan.issue(kbase, vbase, it.r0, it.re, row_bytes, row_stride, sm.a[0], sm.b[0], w);

  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int a = 0; a < 16; ++a) acc[t][a] = 0.f;
  uint32_t tlo[D / 32], thi[D / 32];
  tr_offsets<D>(tlo, thi, l);
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();

  // the tile after `it` is advanced one iteration ahead, after the products are issued, so
  // the walk's scalar work is off the loop head where every wave meets after the barrier
  Tiles nx = it;
  nx.next();
  int buf = 0;
  while (it.valid()) {
    const int valid = min(kT, it.re - it.r0);
    if (nx.valid()) plan.issue(kbase, vbase, nx.r0, nx.re, row_bytes, row_stride, sm.a[buf ^ 1], sm.b[buf ^ 1], w);
    const uint16_t* sk = sm.a[buf];
    const uint16_t* sv = sm.b[buf];
    f32x16 s[NST], dp[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int a = 0; a < 16; ++a) s[st][a] = 0.f, dp[st][a] = 0.f;
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd)
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int row = 32 * (kh + st) + col;
        s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag<D>(sk, row, kd, g), qf[kd], s[st], 0, 0, 0);
        dp[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag<D>(sv, row, kd, g), df[kd], dp[st], 0, 0, 0);
      }
    // dS^T = P^T (dP^T - D); keys past the tile's end get P = 0
    bf16x8 dsb[2 * NST];
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int key = 32 * (kh + st) + 8 * (a >> 2) + 4 * g + (a & 3);
        const float p = key < valid ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][a], scale_log2, -lse2)) : 0.f;
        dsb[2 * st + (a >> 3)][a & 7] = (__bf16)(p * (dp[st][a] - dlt));
      }
    // dQ^T += K^T dS^T, 16 keys per product, K read transposed
#pragma unroll
    for (int kk = 0; kk < 2 * NST; ++kk) {
      bf16x8 kt[D / 32];
      read_tr<D>(kt, tlo, thi, lds_addr(sk + 16 * (2 * kh + kk) * D));
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[t], dsb[kk], acc[t], 0, 0, 0);
    }
    Tiles nn = nx;
    nn.next();
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    buf ^= 1;
    it = nx;
    nx = nn;
  }

  if constexpr (KS == 2) {  // the key halves add
    float* xb = (float*)&sm + (qw * kWave + l) * (D / 2);
    if (kh == 1)
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int a = 0; a < 16; ++a) xb[16 * t + a] = acc[t][a];
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int a = 0; a < 16; ++a) acc[t][a] += xb[16 * t + a];
  }
  if (ok) {
    float* op = dq + ((b * nq + my_q) * heads + h) * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = acc[t][4 * a4 + i] * scale;
        *(f32x4*)(op + 32 * t + 8 * a4 + 4 * g) = x;
      }
  }
}

// ------------------------------------------------------------------ 4. dK, dV
// A workgroup of 4 waves owns 32 * 4 / KS key rows of one key block; with KS = 2 the wave
// pairs (w, w + 2) share 32 keys and split each query tile, adding their sums at the end.
// Grouped (GR): the 4 waves own gp.G key blocks of <= 64 keys (gp.wpb waves each) and walk
// the union of their query blocks; a wave whose block is not kept by a tile's query block
// only helps copy it.  One copy of Q and dO then serves 128 keys instead of 64.
template <int D, int KS, bool GR>
__global__ __launch_bounds__(kNW * kWave, 2) void dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dk, float* __restrict__ dv, int64_t nq, int64_t nk, int heads, int block_q, int block_k,
    const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ row_idx,
    const int32_t* __restrict__ gmask, const int32_t* __restrict__ gcnt, int n_slabs, float scale,
    float scale_log2, Work wk, KeyGroups gp) {
  static_assert(!GR || KS == 1, "grouped key blocks use whole query tiles");
  __shared__ __attribute__((aligned(1024))) Smem<D> sm;
  constexpr int BN = 32 * kNW / KS;
  constexpr int NQS = 2 / KS;  // 32-query steps of a tile per wave
  const int64_t bid = blockIdx.x;
  const int64_t item = work_item(wk, bid);
  if (item >= wk.items) return;
  const int mt = (int)(item % wk.mt_per_b);
  int64_t rest = item / wk.mt_per_b;
  const int kb = (int)(rest % wk.nb);  // key block, or group of key blocks
  rest /= wk.nb;
  const int h = (int)(rest % heads);
  const int64_t b = rest / heads;

  const int l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int col = l & 31, g = l >> 5;
  const int kw = KS == 1 ? (GR ? 0 : w) : (w & 1);
  const int qh = KS == 1 ? 0 : (w >> 1);
  const int row_stride = heads * D;
  const uint32_t row_bytes = 2u * (uint32_t)row_stride;

  // the workgroup's keys [k_lo, k_hi) -- grouped: this wave's 32 keys (possibly none)
  int64_t k_lo, k_hi;
  int lk = 0;  // grouped: the wave's key block within the group
  if constexpr (GR) {
    lk = w / gp.wpb;
    const int64_t kbw = (int64_t)kb * gp.G + lk;
    k_lo = kbw * block_k + (int64_t)(w % gp.wpb) * 32;
    k_hi = min(min((kbw + 1) * block_k, nk), k_lo + 32);
  } else {
    k_lo = (int64_t)kb * block_k + (int64_t)mt * BN;
    k_hi = min(min((int64_t)(kb + 1) * block_k, nk), k_lo + BN);
    if (k_lo >= k_hi) return;
  }

  const int64_t slab = n_slabs == 1 ? 0 : b * heads + h;
  Tiles it;
  if constexpr (GR) {
    const int64_t u = slab * wk.nb + kb;
    it = Tiles{row_idx, (int)(u * gp.cap), (int)(u * gp.cap) + gcnt[u], 0, 0, block_q, (int)nq};
  } else {
    const int64_t c = slab * wk.nb + kb;
    it = Tiles{row_idx, col_ptr[c], col_ptr[c + 1], 0, 0, block_q, (int)nq};
  }
  it.open();
  const uint16_t* qbase = q + (b * nq * heads + h) * (int64_t)D;
  const uint16_t* dobase = dout + (b * nq * heads + h) * (int64_t)D;
  const float* lse_h = lse + (b * heads + h) * nq;
  const float* dl_h = delta + (b * heads + h) * nq;
  // Two waves per SIMD need the kernel within 256 registers: the copy plan and the
  // transposed-read offsets are remade from an opaque lane id where they are used (kept
  // live across the loop they would cost 24 registers).  KS = 1 then spills three dwords,
  // reloaded once per tile; KS = 2 (its query-half merge adds to the pressure) spills a
  // few fragments per tile, and still runs faster than at one wave per SIMD.
  auto lane = [&]() {
    int x = l;
    asm volatile("" : "+v"(x));
    return x;
  };
  // wave 0 stages the tile's lse and D through registers (64 queries, one per lane)
  auto fetch_ld = [&](int r0, int re, float& lv, float& dv_) {
    const int qq = r0 + l;
    lv = qq < re ? lse_h[qq] * kLog2e : INFINITY;
    dv_ = qq < re ? dl_h[qq] : 0.f;
  };

  // this lane's key: B operands K^T and V^T
  const int64_t my_k = k_lo + kw * 32 + col;
  const bool ok = my_k < k_hi;
  bf16x8 kf[D / 16], vf[D / 16];
  {
    // a lane past the keys reads nothing; its address still names a row that exists (a
    // grouped wave past the last key block has k_lo >= nk)
    const int64_t base = ((b * nk + (ok ? my_k : (GR ? 0 : k_lo))) * heads + h) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      kf[s] = __builtin_bit_cast(bf16x8, ok ? *(const u32x4*)(k + base + 16 * s) : u32x4{0, 0, 0, 0});
      vf[s] = __builtin_bit_cast(bf16x8, ok ? *(const u32x4*)(v + base + 16 * s) : u32x4{0, 0, 0, 0});
    }
  }
  float lv = 0.f, dv_ = 0.f;
  if (it.valid()) {
    CopyPlan<D>::issue_lean(qbase, dobase, it.r0, it.re, row_bytes, row_stride, sm.a[0], sm.b[0], w, lane());
    if (w == 0) {
      fetch_ld(it.r0, it.re, lv, dv_);
      sm.lse[0][l] = lv;
      sm.dl[0][l] = dv_;
    }
  }

  f32x16 adk[D / 32], adv[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int a = 0; a < 16; ++a) adk[t][a] = 0.f, adv[t][a] = 0.f;
  wait_vmcnt<0>();
  __syncthreads();

  // the tile after `it` is advanced one iteration ahead (as in the dQ kernel)
  Tiles nx = it;
  nx.next();
  int buf = 0;
  while (it.valid()) {
    if (nx.valid()) {
      // the next tile's lse and D first: a wait for these loads then leaves the copies issued
      // after them in flight (loads complete in order)
      if (w == 0) fetch_ld(nx.r0, nx.re, lv, dv_);
      CopyPlan<D>::issue_lean(qbase, dobase, nx.r0, nx.re, row_bytes, row_stride, sm.a[buf ^ 1], sm.b[buf ^ 1], w,
                              lane());
    }
    const uint16_t* sq = sm.a[buf];
    const uint16_t* sd = sm.b[buf];
    const bool member = !GR || ((gmask[it.e] >> lk) & 1);
#pragma unroll
    for (int qs = 0; qs < NQS; ++qs) {
      if (!member) break;
      const int q32 = 32 * (qh + qs);  // first query of this 32-query step within the tile
      // the fragment rows and lane halves from an opaque lane id, remade at each step: kept
      // live across the loop, their 16 read offsets were spilled, and the reload's wait
      // also waited for the copies of the next tile
      const int ln = lane(), rq = q32 + (ln & 31), gq = ln >> 5;
      // S, then P (fp32, kept in s) and its bf16 copy, then dV^T += dO^T P; rows past the
      // tile's end have lse = +inf, so P = 0 there
      f32x16 s;
#pragma unroll
      for (int a = 0; a < 16; ++a) s[a] = 0.f;
#pragma unroll
      for (int kd = 0; kd < D / 16; ++kd)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag<D>(sq, rq, kd, gq), kf[kd], s, 0, 0, 0);
      bf16x8 pb[2];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 l4 = *(const f32x4*)&sm.lse[buf][q32 + 8 * a4 + 4 * g];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int a = 4 * a4 + i;
          s[a] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[a], scale_log2, -l4[i]));
          pb[a >> 3][a & 7] = (__bf16)s[a];
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 xt[D / 32];
        uint32_t tlo[D / 32], thi[D / 32];
        tr_offsets<D>(tlo, thi, lane());
        read_tr<D>(xt, tlo, thi, lds_addr(sd + (q32 + 16 * kk) * D));
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
          adv[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xt[t], pb[kk], adv[t], 0, 0, 0);
      }
      // dP, then dS = P (dP - D), then dK^T += Q^T dS
      f32x16 dp;
#pragma unroll
      for (int a = 0; a < 16; ++a) dp[a] = 0.f;
#pragma unroll
      for (int kd = 0; kd < D / 16; ++kd)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag<D>(sd, rq, kd, gq), vf[kd], dp, 0, 0, 0);
      bf16x8 db[2];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 d4 = *(const f32x4*)&sm.dl[buf][q32 + 8 * a4 + 4 * g];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int a = 4 * a4 + i;
          db[a >> 3][a & 7] = (__bf16)(s[a] * (dp[a] - d4[i]));
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 xt[D / 32];
        uint32_t tlo[D / 32], thi[D / 32];
        tr_offsets<D>(tlo, thi, lane());
        read_tr<D>(xt, tlo, thi, lds_addr(sq + (q32 + 16 * kk) * D));
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
          adk[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xt[t], db[kk], adk[t], 0, 0, 0);
      }
    }
    if (nx.valid() && w == 0) {
      sm.lse[buf ^ 1][l] = lv;
      sm.dl[buf ^ 1][l] = dv_;
    }
    Tiles nn = nx;
    nn.next();
    wait_vmcnt<0>();
    __syncthreads();
    buf ^= 1;
    it = nx;
    nx = nn;
  }

  if constexpr (KS == 2) {  // the query halves add
    float* xb = (float*)&sm + (kw * kWave + l) * D;
    if (qh == 1)
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int a = 0; a < 16; ++a) xb[16 * t + a] = adk[t][a], xb[D / 2 + 16 * t + a] = adv[t][a];
    __syncthreads();
    if (qh == 1) return;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int a = 0; a < 16; ++a) adk[t][a] += xb[16 * t + a], adv[t][a] += xb[D / 2 + 16 * t + a];
  }
  if (ok) {
    const int64_t off = ((b * nk + my_k) * heads + h) * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 xk, xv;
#pragma unroll
        for (int i = 0; i < 4; ++i) xk[i] = adk[t][4 * a4 + i] * scale, xv[i] = adv[t][4 * a4 + i];
        *(f32x4*)(dk + off + 32 * t + 8 * a4 + 4 * g) = xk;
        *(f32x4*)(dv + off + 32 * t + 8 * a4 + 4 * g) = xv;
      }
  }
}

// ------------------------------------------------------------------ fp32
// One wave per query row (dQ) or key row (dK, dV); lanes over head_dim.
__device__ inline float wave_sum(float x) {
  for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void dq_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                     const float* __restrict__ v, const float* __restrict__ dout,
                                                     const float* __restrict__ lse, const float* __restrict__ delta,
                                                     float* __restrict__ dq, int64_t batch, int64_t nq, int64_t nk,
                                                     int heads, int block_q, int block_k,
                                                     const int32_t* __restrict__ row_ptr,
                                                     const int32_t* __restrict__ col_idx, int n_slabs, int nbq,
                                                     float scale) {
  constexpr int E = D / kWave;  // elements per lane
  const int64_t wid = ((int64_t)blockIdx.x * 256 + threadIdx.x) / kWave;
  if (wid >= batch * heads * nq) return;
  const int l = lane_id();
  const int64_t qi = wid % nq, bh = wid / nq, b = bh / heads;
  const int h = (int)(bh % heads);
  const float* qp = q + ((b * nq + qi) * heads + h) * D;
  const float* dp_ = dout + ((b * nq + qi) * heads + h) * D;
  float qv[E], dov[E], acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) qv[i] = qp[l + kWave * i], dov[i] = dp_[l + kWave * i], acc[i] = 0.f;
  const float ls = lse[bh * nq + qi], dl = delta[bh * nq + qi];
  const int64_t r = (n_slabs == 1 ? 0 : bh) * nbq + qi / block_q;
  for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
    const int64_t k0 = (int64_t)col_idx[e] * block_k, k1 = min(k0 + block_k, nk);
    for (int64_t j = k0; j < k1; ++j) {
      const float* kp = k + ((b * nk + j) * heads + h) * D;
      const float* vp = v + ((b * nk + j) * heads + h) * D;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) s += qv[i] * kp[l + kWave * i], dp += dov[i] * vp[l + kWave * i];
      s = wave_sum(s);
      dp = wave_sum(dp);
      const float ds = expf(s * scale - ls) * (dp - dl);
#pragma unroll
      for (int i = 0; i < E; ++i) acc[i] += ds * kp[l + kWave * i];
    }
  }
  float* op = dq + ((b * nq + qi) * heads + h) * D;
#pragma unroll
  for (int i = 0; i < E; ++i) op[l + kWave * i] = acc[i] * scale;
}

template <int D>
__global__ __launch_bounds__(256) void dkdv_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                       const float* __restrict__ v, const float* __restrict__ dout,
                                                       const float* __restrict__ lse, const float* __restrict__ delta,
                                                       float* __restrict__ dk, float* __restrict__ dv, int64_t batch,
                                                       int64_t nq, int64_t nk, int heads, int block_q, int block_k,
                                                       const int32_t* __restrict__ col_ptr,
                                                       const int32_t* __restrict__ row_idx, int n_slabs, int nbk,
                                                       float scale) {
  constexpr int E = D / kWave;
  const int64_t wid = ((int64_t)blockIdx.x * 256 + threadIdx.x) / kWave;
  if (wid >= batch * heads * nk) return;
  const int l = lane_id();
  const int64_t kj = wid % nk, bh = wid / nk, b = bh / heads;
  const int h = (int)(bh % heads);
  const float* kp = k + ((b * nk + kj) * heads + h) * D;
  const float* vp = v + ((b * nk + kj) * heads + h) * D;
  float kv[E], vv[E], ak[E], av[E];
#pragma unroll
  for (int i = 0; i < E; ++i) kv[i] = kp[l + kWave * i], vv[i] = vp[l + kWave * i], ak[i] = 0.f, av[i] = 0.f;
  const int64_t c = (n_slabs == 1 ? 0 : bh) * nbk + kj / block_k;
  for (int32_t e = col_ptr[c]; e < col_ptr[c + 1]; ++e) {
    const int64_t q0 = (int64_t)row_idx[e] * block_q, q1 = min(q0 + block_q, nq);
    for (int64_t i = q0; i < q1; ++i) {
      const float* qp = q + ((b * nq + i) * heads + h) * D;
      const float* dp_ = dout + ((b * nq + i) * heads + h) * D;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int x = 0; x < E; ++x) s += qp[l + kWave * x] * kv[x], dp += dp_[l + kWave * x] * vv[x];
      s = wave_sum(s);
      dp = wave_sum(dp);
      const float p = expf(s * scale - lse[bh * nq + i]);
      const float ds = p * (dp - delta[bh * nq + i]);
#pragma unroll
      for (int x = 0; x < E; ++x) av[x] += p * dp_[l + kWave * x], ak[x] += ds * qp[l + kWave * x];
    }
  }
  float* okp = dk + ((b * nk + kj) * heads + h) * D;
  float* ovp = dv + ((b * nk + kj) * heads + h) * D;
#pragma unroll
  for (int x = 0; x < E; ++x) okp[l + kWave * x] = ak[x] * scale, ovp[l + kWave * x] = av[x];
}

Work make_work(int64_t batch, int heads, int64_t n, int block, int rows_per_wg) {
  Work wk;
  wk.nb = (int)((n + block - 1) / block);
  wk.mt_per_b = (block + rows_per_wg - 1) / rows_per_wg;
  wk.items = batch * heads * (int64_t)wk.nb * wk.mt_per_b;
  wk.per_xcd = (wk.items + 7) / 8;
  return wk;
}

}  // namespace

// Grouped dK, dV (bf16, key blocks of <= 64 keys): G = 4 / wpb key blocks per 4-wave
// workgroup when that still leaves two workgroups per CU; G = 0 means ungrouped.
struct KeyGroupPlan {
  int G = 0, wpb = 1, n_groups = 0;
  int64_t lists = 0;
};

KeyGroupPlan plan_key_groups(const AttnBwdArgs& a) {
  KeyGroupPlan p;
  const int64_t nbq = (a.nq + a.block_q - 1) / a.block_q, nbk = (a.nk + a.block_k - 1) / a.block_k;
  if (a.dtype != 1 || a.block_k > 64) return p;
  const int wpb = (a.block_k + 31) / 32, G = kNW / wpb;
  const int64_t n_groups = (nbk + G - 1) / G;
  const int64_t lists = (int64_t)a.n_slabs * n_groups;
  if (a.batch * a.heads * n_groups < 512 || lists * nbq > 0x7fffffff) return p;
  p.G = G;
  p.wpb = wpb;
  p.n_groups = (int)n_groups;
  p.lists = lists;
  return p;
}

size_t attn_bwd_workspace(const AttnBwdArgs& a) {
  const int64_t nbq = (a.nq + a.block_q - 1) / a.block_q, nbk = (a.nk + a.block_k - 1) / a.block_k;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const KeyGroupPlan kg = plan_key_groups(a);
  return al(4 * (size_t)(a.batch * a.heads * a.nq)) + al(4 * (size_t)(a.n_slabs * nbk)) +
         al(4 * (size_t)(a.n_slabs * nbk + 1)) + al(4 * (size_t)(a.n_slabs * nbq * nbk)) +
         (kg.G ? 2 * al(4 * (size_t)(kg.lists * nbq)) + al(4 * (size_t)kg.lists) : 0);
}

hipError_t launch_attn_bwd(const AttnBwdArgs& a, void* workspace, hipStream_t stream) {
  const int nbq = (int)((a.nq + a.block_q - 1) / a.block_q), nbk = (int)((a.nk + a.block_k - 1) / a.block_k);
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  char* ws = (char*)workspace;
  float* delta = (float*)ws;
  ws += al(4 * (size_t)(a.batch * a.heads * a.nq));
  int32_t* cnt = (int32_t*)ws;
  ws += al(4 * (size_t)(a.n_slabs * nbk));
  int32_t* col_ptr = (int32_t*)ws;
  ws += al(4 * (size_t)(a.n_slabs * nbk + 1));
  int32_t* row_idx = (int32_t*)ws;
  ws += al(4 * (size_t)(a.n_slabs * nbq * nbk));
  const KeyGroupPlan kg = plan_key_groups(a);
  KeyGroups kgp{1, 1, 0};
  int32_t *gidx = nullptr, *gmask = nullptr, *gcnt = nullptr;
  if (kg.G) {
    gidx = (int32_t*)ws;
    ws += al(4 * (size_t)(kg.lists * nbq));
    gmask = (int32_t*)ws;
    ws += al(4 * (size_t)(kg.lists * nbq));
    gcnt = (int32_t*)ws;
    kgp = KeyGroups{kg.G, kg.wpb, nbq};
  }

  const bool bf16 = a.dtype == 1;
  const int64_t rows = a.batch * a.nq;
  const int64_t threads = rows * a.heads * a.head_dim / 8;
  const dim3 g1((unsigned)((threads + 255) / 256));
  if (a.head_dim == 64)
    hipLaunchKernelGGL(delta_kernel<8>, g1, dim3(256), 0, stream, (const uint8_t*)a.o, (const uint8_t*)a.dout,
                       (int)bf16, rows, a.heads, a.head_dim, a.nq, delta);
  else
    hipLaunchKernelGGL(delta_kernel<16>, g1, dim3(256), 0, stream, (const uint8_t*)a.o, (const uint8_t*)a.dout,
                       (int)bf16, rows, a.heads, a.head_dim, a.nq, delta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(csc_kernel, dim3((unsigned)a.n_slabs), dim3(kCscThreads), 0, stream, a.row_ptr, a.col_idx,
                     nbq, nbk, (int64_t)a.n_slabs, cnt, col_ptr, row_idx);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  if (!bf16) {
    const int64_t wq = a.batch * a.heads * a.nq, wkk = a.batch * a.heads * a.nk;
    const dim3 gq((unsigned)((wq * kWave + 255) / 256)), gk((unsigned)((wkk * kWave + 255) / 256));
    auto go = [&](auto dqk, auto dkk) {
      hipLaunchKernelGGL(dqk, gq, dim3(256), 0, stream, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                         (const float*)a.dout, a.lse, delta, a.dq, a.batch, a.nq, a.nk, a.heads, a.block_q,
                         a.block_k, a.row_ptr, a.col_idx, a.n_slabs, nbq, a.scale);
      hipLaunchKernelGGL(dkk, gk, dim3(256), 0, stream, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                         (const float*)a.dout, a.lse, delta, a.dk, a.dv, a.batch, a.nq, a.nk, a.heads, a.block_q,
                         a.block_k, col_ptr, row_idx, a.n_slabs, nbk, a.scale);
    };
    if (a.head_dim == 64) go(dq_f32_kernel<64>, dkdv_f32_kernel<64>);
    else go(dq_f32_kernel<128>, dkdv_f32_kernel<128>);
    return hipGetLastError();
  }

  const float sl2 = a.scale * kLog2e;
  const int ksq = a.block_q <= 64 ? 2 : 1, ksk = a.block_k <= 64 ? 2 : 1;
  Work wq = make_work(a.batch, a.heads, a.nq, a.block_q, 32 * kNW / ksq);
  Work wkv = make_work(a.batch, a.heads, a.nk, a.block_k, 32 * kNW / ksk);
  wq.chunk = wkv.chunk = xcd_run(a.nk, a.head_dim, 2);
  if (kg.G) {  // the union of each group's query blocks, from the CSC view
    if ((e = launch_group_union(col_ptr, row_idx, nbk, kg.lists, kg.G, kg.n_groups, 1, nbq, gidx, gmask, gcnt,
                                stream)) != hipSuccess)
      return e;
    wkv.nb = kg.n_groups;
    wkv.mt_per_b = 1;
    wkv.items = a.batch * a.heads * (int64_t)kg.n_groups;
    wkv.per_xcd = (wkv.items + 7) / 8;
  }
  auto lq = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)(wq.per_xcd * 8)), dim3(kNW * kWave), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout,
                       a.lse, delta, a.dq, a.nq, a.nk, a.heads, a.block_q, a.block_k, a.row_ptr, a.col_idx,
                       a.n_slabs, a.scale, sl2, wq);
  };
  auto lk = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)(wkv.per_xcd * 8)), dim3(kNW * kWave), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout,
                       a.lse, delta, a.dk, a.dv, a.nq, a.nk, a.heads, a.block_q, a.block_k, col_ptr,
                       kg.G ? gidx : row_idx, gmask, gcnt, a.n_slabs, a.scale, sl2, wkv, kgp);
  };
  if (a.head_dim == 64) {
    ksq == 2 ? lq(dq_kernel<64, 2>) : lq(dq_kernel<64, 1>);
    if (kg.G) lk(dkdv_kernel<64, 1, true>);
    else ksk == 2 ? lk(dkdv_kernel<64, 2, false>) : lk(dkdv_kernel<64, 1, false>);
  } else {
    ksq == 2 ? lq(dq_kernel<128, 2>) : lq(dq_kernel<128, 1>);
    if (kg.G) lk(dkdv_kernel<128, 1, true>);
    else ksk == 2 ? lk(dkdv_kernel<128, 2, false>) : lk(dkdv_kernel<128, 1, false>);
  }
  return hipGetLastError();
}

}  // namespace vsa

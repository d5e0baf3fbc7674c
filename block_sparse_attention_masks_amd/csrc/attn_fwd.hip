// Block-sparse attention forward: exact softmax(Q K^T * scale) V over the key
// blocks a CSR mask keeps (SPADE summary, gist.science/ja/paper/2608.03335, "The
// solution" part 3: head-wise sparse attention on the kept blocks only; the
// pages' masks decide which blocks are kept).
//
// bf16 path (matrix cores).  A workgroup of 4 waves owns 128 query rows of one
// (batch, head, query block); each wave owns 32 of them, held in registers as
// the B operand of S^T = K Q^T.  The kept key blocks are walked as one stream of
// 64-key tiles:
//   * tile t+1 is fetched from HBM into registers (16-byte loads) while tile t is
//     computed from LDS; the registers are then written to the other half of a
//     double-buffered LDS stage, so each tile costs one barrier;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (M = keys, N = queries, K = head
//     dim): the accumulator gives each lane one query and 16 keys, so the row max
//     and row sum are in-lane plus one exchange between the half-waves;
//   * online softmax in the log2 domain with a lazy reference maximum: the
//     output is rescaled only when a row's maximum grows by more than 2^8, which
//     keeps every exponent <= 2^8 and leaves the normalised result unchanged;
//   * O^T += V^T P^T on the same instruction (M = head dim, N = queries, K =
//     keys), P rounded to bf16; the row sum adds the rounded values, so the
//     weights applied to V are exactly normalised.  V stays row-major in LDS; ds_read_b64_tr_b16
//     delivers each lane its 8 keys of one head-dim column.  The key order inside
//     each 16-key group follows the S accumulator layout (lane half g holds keys
//     4g..4g+3 and 8+4g..8+4g+3), so P feeds the product without any shuffle.
// Ragged key tails are masked with -inf; query rows past the block or the
// sequence are computed but never stored.  A row with no kept block writes 0
// and lse = -inf.
//
// fp32 path: the same definition evaluated with fp32 FMA on the vector units,
// one thread per query row (used for small fp32 problems).
#include <math.h>

#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;      // query rows per workgroup
constexpr int kBN = 64;       // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale slack (exponents stay <= 2^8)

struct Work {
  int64_t items, per_xcd;
  int nbq, mt_per_qb;
};

// LDS row pitches (elements).  K rows shift by 4 banks (conflict-free 16-byte
// reads of 16 consecutive rows); V rows shift by 16 banks (conflict-free
// transposed 8-byte reads of 4 consecutive rows x 64 bytes).
template <int D> struct Pitch;
template <> struct Pitch<128> { static constexpr int K = 136, V = 160; };
template <> struct Pitch<64> { static constexpr int K = 72, V = 96; };

template <int D>
struct Smem {
  uint16_t k[2][kBN * Pitch<D>::K];
  uint16_t v[2][kBN * Pitch<D>::V];
};

// Stream of 64-key tiles over the kept blocks of one CSR row (wave-uniform).
struct TileIter {
  const int32_t* col;
  int e, e1;
  int64_t k0, ke;
  int block_k;
  int64_t nk;
  __device__ bool valid() const { return e < e1; }
  __device__ void open() {  // position on the first tile of block col[e]
    if (e < e1) {
      const int64_t ks = (int64_t)col[e] * block_k;
      k0 = ks;
      ke = min(ks + block_k, nk);
    }
  }
  __device__ void next() {
    k0 += kBN;
    if (k0 >= ke) {
      ++e;
      open();
    }
  }
};

// Value held by lane l ^ 32 (the other half-wave), via v_permlane32_swap (no LDS).
__device__ inline float xchg32(float x, int g) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(g == 0 ? r[1] : r[0]);
}

template <int D, int KS>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    int64_t nq, int64_t nk, int heads, int block_q, int block_k,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int n_slabs,
    float scale_log2, Work wk) {
  __shared__ __attribute__((aligned(16))) Smem<D> sm;
  constexpr int kPer = kBN * D / 8 / kThreads;  // 16-byte chunks per thread per tensor
  // KS = 1: the 4 waves own 32 query rows each and all 64 keys of every tile.
  // KS = 2 (query blocks of <= 64 rows): waves w and w+2 own the same 32 rows and
  // split every tile's keys in halves; their softmax states merge at the end.
  constexpr int BM = kBM / KS;   // query rows per workgroup
  constexpr int NST = 2 / KS;    // 32-key sub-tiles per wave per tile

  // XCD-aware mapping: workgroups are dealt round-robin to the 8 XCDs; give each
  // XCD a contiguous range of work items so that the query tiles of one query
  // block (which read the same K/V) share an L2.
  const int64_t bid = blockIdx.x;
  const int64_t item = (bid % 8) * wk.per_xcd + bid / 8;
  if (item >= wk.items) return;
  const int mt = (int)(item % wk.mt_per_qb);
  int64_t rest = item / wk.mt_per_qb;
  const int qb = (int)(rest % wk.nbq);
  rest /= wk.nbq;
  const int h = (int)(rest % heads);
  const int64_t b = rest / heads;

  const int64_t q_lo = (int64_t)qb * block_q + (int64_t)mt * BM;
  const int64_t q_hi = min(min((int64_t)(qb + 1) * block_q, nq), q_lo + BM);
  if (q_lo >= q_hi) return;

  const int tid = threadIdx.x, w = tid / kWave, l = lane_id();
  const int col = l & 31, g = l >> 5;
  const int qw = KS == 1 ? w : (w & 1);   // this wave's 32-row query group
  const int kh = KS == 1 ? 0 : (w >> 1);  // this wave's key half (KS = 2)
  const int row_stride = heads * D;  // elements between tokens (validated < 2^31 / 64)

  const int64_t slab = n_slabs == 1 ? 0 : b * heads + h;
  const int64_t r = slab * wk.nbq + qb;
  TileIter it{col_idx, row_ptr[r], row_ptr[r + 1], 0, 0, block_k, nk};
  it.open();

  const uint16_t* kbase = k + (b * nk * heads + h) * (int64_t)D;
  const uint16_t* vbase = v + (b * nk * heads + h) * (int64_t)D;

  // This thread stages chunks tid + 256 i of each tile: key row krow0 + kRowStep*i,
  // head-dim columns d8 .. d8+7 (the same for every tile).
  constexpr int kRowStep = kThreads / (D / 8);
  const int krow0 = tid / (D / 8), d8 = (tid % (D / 8)) * 8;
  const int goff0 = krow0 * row_stride + d8;
  const int soff_k = krow0 * Pitch<D>::K + d8, soff_v = krow0 * Pitch<D>::V + d8;
  u32x4 kreg[kPer], vreg[kPer];
  auto load = [&](const TileIter& t) {
    const uint16_t* kb = kbase + t.k0 * row_stride + goff0;
    const uint16_t* vb = vbase + t.k0 * row_stride + goff0;
    const int nv = (int)min((int64_t)kBN, t.ke - t.k0);
    if (nv == kBN) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        kreg[i] = *(const u32x4*)(kb + i * kRowStep * row_stride);
        vreg[i] = *(const u32x4*)(vb + i * kRowStep * row_stride);
      }
    } else {  // ragged tail: rows past the block read as zero
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const bool ok = krow0 + i * kRowStep < nv;
        kreg[i] = ok ? *(const u32x4*)(kb + i * kRowStep * row_stride) : u32x4{0, 0, 0, 0};
        vreg[i] = ok ? *(const u32x4*)(vb + i * kRowStep * row_stride) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store = [&](int bufi) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      *(u32x4*)(sm.k[bufi] + soff_k + i * kRowStep * Pitch<D>::K) = kreg[i];
      *(u32x4*)(sm.v[bufi] + soff_v + i * kRowStep * Pitch<D>::V) = vreg[i];
    }
  };
  if (it.valid()) {
    load(it);
    store(0);
  }

  // Q fragments (B operand of S^T = K Q^T): query col, dims 16*s + 8*g .. +7.
  const int64_t my_q = q_lo + qw * 32 + col;
  bf16x8 qf[D / 16];
  {
    const bool ok = my_q < q_hi;
    const uint16_t* qp = q + ((b * nq + (ok ? my_q : q_lo)) * heads + h) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 u = ok ? *(const u32x4*)(qp + 16 * s) : u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, u);
    }
  }

  f32x16 acc_o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int a = 0; a < 16; ++a) acc_o[t][a] = 0.f;
  float m_ref = -INFINITY, l_run = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  // transposed-read lane address inside a V tile: key row 4g + j, columns
  // 16*((l/16)%2) + 4c (plus 32t and 16kk rows per product step)
  const int vt_off = (4 * g + ((l & 15) >> 2)) * Pitch<D>::V + 16 * ((l >> 4) & 1) + 4 * (l & 3);
  const int k_off = col * Pitch<D>::K + 8 * g;

  // One 64-key tile: S^T = K Q^T, online softmax, O^T += V^T P^T.  `valid` < 64
  // only for the ragged last tile of a block.
  auto tile = [&](const uint16_t* sk, const uint16_t* sv, int valid) {
    f32x16 s[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int a = 0; a < 16; ++a) s[st][a] = 0.f;
    {
      // K fragments are read kLook steps ahead of the products that use them
      constexpr int kSteps = D / 16, kLook = 2;
      const uint16_t* kp = sk + k_off + 32 * kh * Pitch<D>::K;
      bf16x8 fr[kSteps][NST];
#pragma unroll
      for (int kd = 0; kd < kLook; ++kd)
#pragma unroll
        for (int st = 0; st < NST; ++st)
          fr[kd][st] = *(const bf16x8*)(kp + 32 * st * Pitch<D>::K + 16 * kd);
#pragma unroll
      for (int kd = 0; kd < kSteps; ++kd) {
        if (kd + kLook < kSteps) {
#pragma unroll
          for (int st = 0; st < NST; ++st)
            fr[kd + kLook][st] = *(const bf16x8*)(kp + 32 * st * Pitch<D>::K + 16 * (kd + kLook));
        }
#pragma unroll
        for (int st = 0; st < NST; ++st)
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[kd][st], qf[kd], s[st], 0, 0, 0);
      }
    }
    if (valid < kBN) {
      // a real branch (kept out of the full-tile path): keys past the tail score -inf
      asm volatile("" ::: "memory");
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const int key = 32 * (kh + st) + 8 * (a >> 2) + 4 * g + (a & 3);
          if (key >= valid) s[st][a] = -INFINITY;
        }
    }
    float mx = s[0][0];
    if constexpr (NST == 2) {
#pragma unroll
      for (int a = 0; a < 16; ++a) mx = fmaxf(fmaxf(mx, s[0][a]), s[1][a]);  // v_max3
    } else {
#pragma unroll
      for (int a = 1; a < 16; a += 2) mx = fmaxf(fmaxf(mx, s[0][a]), s[0][a + 1 < 16 ? a + 1 : a]);
    }
    mx = fmaxf(mx, xchg32(mx, g)) * scale_log2;
    const bool grow = mx > m_ref + kRescaleLog2;
    if (__ballot(grow)) {
      // a real branch: keeps the compiler from turning the rare rescale into an
      // unconditional multiply by a selected factor
      asm volatile("" ::: "memory");
      const float m_new = grow ? mx : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int a = 0; a < 16; ++a) acc_o[t][a] *= alpha;
    }
    // a wave whose keys so far were all masked has m_ref = -inf: its weights are 0
    const float m_use = KS == 1 ? m_ref : (m_ref == -INFINITY ? 0.f : m_ref);
    bf16x8 pf[2 * NST];
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int a = 0; a < 16; ++a)
        pf[2 * st + (a >> 3)][a & 7] =
            (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[st][a], scale_log2, -m_use));
    // row sum of the rounded weights (so the weights applied to V sum to exactly 1)
    float psum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2 * NST; ++kk) {
      const bf16x2* pp = (const bf16x2*)&pf[kk];
#pragma unroll
      for (int i = 0; i < 4; ++i) psum = __builtin_amdgcn_fdot2_f32_bf16(pp[i], ones, psum, false);
    }
    l_run += psum;

    // O^T += V^T P^T; A operand (V^T) by transposed LDS reads: lane (j = (l%16)/4,
    // c = l%4) addresses key row 16kk+4g+j (+8 for the second half) at head-dim
    // columns 32t + 16*((l/16)%2) + 4c .. +3.
#pragma unroll
    for (int kk = 0; kk < 2 * NST; ++kk) {
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        const uint16_t* p0 = sv + vt_off + 16 * (2 * kh + kk) * Pitch<D>::V + 32 * t;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (s16x4 __attribute__((address_space(3)))*)(p0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (s16x4 __attribute__((address_space(3)))*)(p0 + 8 * Pitch<D>::V));
        const s16x4 vv[2] = {lo, hi};
        const bf16x8 vf = __builtin_bit_cast(bf16x8, vv);
        acc_o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk], acc_o[t], 0, 0, 0);
      }
    }
  };
  __syncthreads();

  int buf = 0;
  while (it.valid()) {
    const int valid = (int)min((int64_t)kBN, it.ke - it.k0);
    TileIter nx = it;
    nx.next();
    if (nx.valid()) load(nx);
    tile(sm.k[buf], sm.v[buf], valid);
    if (nx.valid()) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    it = nx;
  }

  // ---- epilogue
  if constexpr (KS == 2) {
    // merge the two key halves: waves 2, 3 hand (m, l, O) to waves 0, 1 through LDS
    float* xb = (float*)&sm + (qw * kWave + l) * (2 + D / 2);
    if (kh == 1) {
      xb[0] = m_ref;
      xb[1] = l_run;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int a = 0; a < 16; ++a) xb[2 + 16 * t + a] = acc_o[t][a];
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = xb[0], l1 = xb[1];
    const float mm = fmaxf(m_ref, m1);
    const float a0 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - mm);
    const float a1 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
    l_run = l_run * a0 + l1 * a1;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int a = 0; a < 16; ++a) acc_o[t][a] = acc_o[t][a] * a0 + xb[2 + 16 * t + a] * a1;
    m_ref = mm;
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (my_q < q_hi) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = o + ((b * nq + my_q) * heads + h) * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = 32 * t + 8 * a4 + 4 * g;
        bf16x4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(acc_o[t][4 * a4 + i] * inv);
        *(bf16x4*)(op + d) = ov;
      }
    if (lse != nullptr && g == 0)
      lse[(b * heads + h) * nq + my_q] =
          l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * 0.6931471805599453f : -INFINITY;
  }
}

// fp32: one thread per (batch, head, query); plain online softmax over the kept keys.
template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int64_t batch, int64_t nq, int64_t nk,
    int heads, int block_q, int block_k, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, int n_slabs, int nbq, float scale) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= batch * heads * nq) return;
  const int64_t tq = gid % nq;
  const int h = (int)((gid / nq) % heads);
  const int64_t b = gid / (nq * heads);
  const int64_t stride = (int64_t)heads * D;
  float qv[D], acc[D];
  const float* qp = q + (b * nq + tq) * stride + (int64_t)h * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = qp[d];
    acc[d] = 0.f;
  }
  float m = -INFINITY, lsum = 0.f;
  const int64_t slab = n_slabs == 1 ? 0 : b * heads + h;
  const int64_t r = slab * nbq + tq / block_q;
  for (int e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
    const int64_t ks = (int64_t)col_idx[e] * block_k, ke = min(ks + block_k, nk);
    for (int64_t kt = ks; kt < ke; ++kt) {
      const float* kp = k + (b * nk + kt) * stride + (int64_t)h * D;
      const float* vp = v + (b * nk + kt) * stride + (int64_t)h * D;
      float sdot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) sdot = fmaf(qv[d], kp[d], sdot);
      sdot *= scale;
      const float mn = fmaxf(m, sdot);
      const float al = expf(m - mn), p = expf(sdot - mn);
      lsum = lsum * al + p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vp[d], acc[d] * al);
      m = mn;
    }
  }
  float* op = o + (b * nq + tq) * stride + (int64_t)h * D;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
  if (lse != nullptr) lse[(b * heads + h) * nq + tq] = lsum > 0.f ? m + logf(lsum) : -INFINITY;
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream) {
  const int nbq = (int)((a.nq + a.block_q - 1) / a.block_q);
  if (a.dtype == 0) {
    const int64_t n = a.batch * a.heads * a.nq;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (a.head_dim == 64)
      hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, grid, dim3(256), 0, stream, (const float*)a.q,
                         (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.batch, a.nq,
                         a.nk, a.heads, a.block_q, a.block_k, a.row_ptr, a.col_idx, a.n_slabs, nbq,
                         a.scale);
    else
      hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, grid, dim3(256), 0, stream, (const float*)a.q,
                         (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.batch, a.nq,
                         a.nk, a.heads, a.block_q, a.block_k, a.row_ptr, a.col_idx, a.n_slabs, nbq,
                         a.scale);
    return hipGetLastError();
  }
  const float sl2 = a.scale * kLog2e;
  const int ks = a.block_q <= kBM / 2 ? 2 : 1;
  Work wk;
  wk.nbq = nbq;
  wk.mt_per_qb = (a.block_q + kBM / ks - 1) / (kBM / ks);
  wk.items = a.batch * a.heads * (int64_t)nbq * wk.mt_per_qb;
  wk.per_xcd = (wk.items + 7) / 8;
  const dim3 grid((unsigned)(wk.per_xcd * 8));
  auto launch = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.nq, a.nk,
                       a.heads, a.block_q, a.block_k, a.row_ptr, a.col_idx, a.n_slabs, sl2, wk);
  };
  if (a.head_dim == 64)
    ks == 2 ? launch(attn_fwd_bf16_kernel<64, 2>) : launch(attn_fwd_bf16_kernel<64, 1>);
  else
    ks == 2 ? launch(attn_fwd_bf16_kernel<128, 2>) : launch(attn_fwd_bf16_kernel<128, 1>);
  return hipGetLastError();
}

}  // namespace vsa

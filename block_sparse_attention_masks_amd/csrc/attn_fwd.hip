// Block-sparse attention forward: exact softmax(Q K^T * scale) V over the key
// blocks a CSR mask keeps (SPADE summary, gist.science/ja/paper/2608.03335, "The
// solution" part 3: head-wise sparse attention on the kept blocks only; the
// pages' masks decide which blocks are kept).
//
// bf16 path (matrix cores).  A workgroup of 4 waves owns 128 query rows of one
// (batch, head, query block); each wave owns 32 of them.  For every kept key
// block the workgroup walks 64-key tiles:
//   * K and V tiles go HBM -> LDS (16-byte loads); V is stored transposed,
//     V^T[d][key], with the keys of each 16-key group permuted (quads 1 and 2
//     swapped) so that the probabilities come out of the S accumulators in
//     exactly the operand layout of the P V product;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (M = keys, N = queries, K = head
//     dim).  The accumulator of a 32x32 tile gives each lane one query column
//     and 16 keys, so the row max / row sum are in-lane plus one exchange
//     between the two half-waves;
//   * online softmax in the log2 domain (scale * log2(e) folded in), running max
//     and sum per query, rescale of the output accumulator;
//   * O^T += V^T P^T on the same instruction (M = head dim, N = queries, K =
//     keys), P rounded to bf16.
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
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;      // query rows per workgroup
constexpr int kBN = 64;       // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kKPad = 8;      // bf16 padding per K row in LDS
constexpr int kVPad = 8;      // bf16 padding per V^T row in LDS
constexpr float kLog2e = 1.4426950408889634f;

struct Work {
  int64_t items, per_xcd;
  int nbq, mt_per_qb;
};

// Position of key `o` (0..15 inside a 16-key group) in the V^T row: quads 1 and 2
// trade places.  Lane half g of the P V product holds keys {4g..4g+3, 8+4g..8+4g+3}
// of the group as its 8 consecutive operand elements.
__device__ inline int vt_slot(int o) {
  const int q4 = o >> 2, r4 = o & 3;
  const int pq = (q4 == 1) ? 2 : (q4 == 2 ? 1 : q4);
  return pq * 4 + r4;
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    int64_t nq, int64_t nk, int heads, int block_q, int block_k,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int n_slabs,
    float scale_log2, Work wk) {
  __shared__ __attribute__((aligned(16))) uint16_t sk[kBN][D + kKPad];
  __shared__ __attribute__((aligned(16))) uint16_t svt[D][kBN + kVPad];

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

  const int64_t q_lo = (int64_t)qb * block_q + (int64_t)mt * kBM;
  const int64_t q_hi = min(min((int64_t)(qb + 1) * block_q, nq), q_lo + kBM);
  if (q_lo >= q_hi) return;

  const int tid = threadIdx.x, w = tid / kWave, l = lane_id();
  const int col = l & 31, g = l >> 5;
  const int64_t row_stride = (int64_t)heads * D;  // elements between tokens

  // Q fragments (B operand of S^T = K Q^T): query col, dims 16*s + 8*g .. +7.
  const int64_t my_q = q_lo + w * 32 + col;
  bf16x8 qf[D / 16];
  {
    const bool ok = my_q < q_hi;
    const uint16_t* qp = q + ((b * nq + (ok ? my_q : q_lo)) * heads + h) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      uint4 u = ok ? *(const uint4*)(qp + 16 * s) : make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(bf16x8, u);
    }
  }

  f32x16 acc_o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int a = 0; a < 16; ++a) acc_o[t][a] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int64_t slab = n_slabs == 1 ? 0 : b * heads + h;
  const int64_t r = slab * wk.nbq + qb;
  const int e0 = row_ptr[r], e1 = row_ptr[r + 1];

  const uint16_t* kbase = k + (b * nk * heads + h) * (int64_t)D;
  const uint16_t* vbase = v + (b * nk * heads + h) * (int64_t)D;

  for (int e = e0; e < e1; ++e) {
    const int j = col_idx[e];
    const int64_t ks = (int64_t)j * block_k;
    const int64_t ke = min(ks + block_k, nk);
    for (int64_t k0 = ks; k0 < ke; k0 += kBN) {
      // ---- stage K and V^T tiles in LDS
      constexpr int kChunks = kBN * D / 8;  // 16-byte chunks per tile
#pragma unroll
      for (int c = tid; c < kChunks; c += kThreads) {
        const int kr = c / (D / 8), d8 = (c % (D / 8)) * 8;
        const int64_t key = k0 + kr;
        uint4 ku = make_uint4(0, 0, 0, 0), vu = make_uint4(0, 0, 0, 0);
        if (key < ke) {
          ku = *(const uint4*)(kbase + key * row_stride + d8);
          vu = *(const uint4*)(vbase + key * row_stride + d8);
        }
        *(uint4*)&sk[kr][d8] = ku;
        const int slot = (kr & ~15) + vt_slot(kr & 15);
        const uint16_t* vh = (const uint16_t*)&vu;
#pragma unroll
        for (int i = 0; i < 8; ++i) svt[d8 + i][slot] = vh[i];
      }
      __syncthreads();

      // ---- S^T = K Q^T for two 32-key sub-tiles
      f32x16 s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int a = 0; a < 16; ++a) s[st][a] = 0.f;
#pragma unroll
        for (int kd = 0; kd < D / 16; ++kd) {
          const bf16x8 af = *(const bf16x8*)&sk[32 * st + col][16 * kd + 8 * g];
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[kd], s[st], 0, 0, 0);
        }
      }

      // ---- online softmax (log2 domain)
      const int valid = (int)min((int64_t)kBN, ke - k0);
      float mt_ = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const int key = 32 * st + 8 * (a >> 2) + 4 * g + (a & 3);
          const float x = key < valid ? s[st][a] * scale_log2 : -INFINITY;
          s[st][a] = x;
          mt_ = fmaxf(mt_, x);
        }
      mt_ = fmaxf(mt_, __shfl_xor(mt_, 32, kWave));
      const float m_new = fmaxf(m_run, mt_);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float psum = 0.f;
      bf16x8 pf[4];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const float p = __builtin_amdgcn_exp2f(s[st][a] - m_new);
          psum += p;
          pf[2 * st + (a >> 3)][a & 7] = (__bf16)p;
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int a = 0; a < 16; ++a) acc_o[t][a] *= alpha;

      // ---- O^T += V^T P^T
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 vf = *(const bf16x8*)&svt[32 * t + col][16 * kk + 8 * g];
          acc_o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk], acc_o[t], 0, 0, 0);
        }
      __syncthreads();
    }
  }

  // ---- epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (my_q < q_hi) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = o + ((b * nq + my_q) * heads + h) * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = 32 * t + 8 * a4 + 4 * g;
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(acc_o[t][4 * a4 + i] * inv);
        *(bf16x4*)(op + d) = ov;
      }
    if (lse != nullptr && g == 0)
      lse[(b * heads + h) * nq + my_q] =
          l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.6931471805599453f : -INFINITY;
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
  Work wk;
  wk.nbq = nbq;
  wk.mt_per_qb = (a.block_q + kBM - 1) / kBM;
  wk.items = a.batch * a.heads * (int64_t)nbq * wk.mt_per_qb;
  wk.per_xcd = (wk.items + 7) / 8;
  const dim3 grid((unsigned)(wk.per_xcd * 8));
  const float sl2 = a.scale * kLog2e;
  if (a.head_dim == 64)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, grid, dim3(kThreads), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.o, a.lse, a.nq, a.nk, a.heads, a.block_q, a.block_k,
                       a.row_ptr, a.col_idx, a.n_slabs, sl2, wk);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, grid, dim3(kThreads), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.o, a.lse, a.nq, a.nk, a.heads, a.block_q, a.block_k,
                       a.row_ptr, a.col_idx, a.n_slabs, sl2, wk);
  return hipGetLastError();
}

}  // namespace vsa

// SICS block scores: the sum of intra-block cosine similarities (SPADE summary,
// gist.science/ja/paper/2608.03335, "The solution" part 2), per (batch, head,
// block) of a token tensor.
//
// Over all ordered token pairs of a block, sum_{i,j} cos(x_i, x_j) equals
// |sum_i x_i / |x_i||^2, so one pass over the rows suffices: HBM-bound, like the
// NABLA pooling.  A workgroup owns one block and 64 consecutive 8-element vectors
// of the token row (4 heads at head_dim 128); its 8 waves take every 8th row of the
// block.  Per row, the D / 8 lanes that hold one head's row reduce its squared norm
// with DPP moves and each adds its slice of the unit row to an fp64
// accumulator; at the end the waves' accumulators are summed through LDS and the
// lanes of each head reduce the squared norm.  A zero row has no direction and
// adds nothing.  Everything after the bf16/fp32 load is fp64.
#include "vsa_internal.h"

namespace vsa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes read once: a streaming (nontemporal) load, which does not displace cached lines
__device__ inline uint4 load_stream(const uint8_t* p) {
  const u32x4 r = __builtin_nontemporal_load((const u32x4*)p);
  return uint4{r.x, r.y, r.z, r.w};
}

// 8 elements widened to fp64: the 16 bytes a (8 bf16) or a then c (8 fp32).
template <bool BF16>
__device__ inline void widen8(const uint4& a, const uint4& c, double* x) {
  if constexpr (BF16) {
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = (double)__uint_as_float(w[i] << 16);
      x[2 * i + 1] = (double)__uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (double)__uint_as_float(w[i]);
  }
}

// One DPP move of a double within each 16-lane row (CTRL: the DPP control code).
template <int CTRL>
__device__ inline double dpp(double v) {
  const int2 u = __builtin_bit_cast(int2, v);
  const int lo = __builtin_amdgcn_update_dpp(0, u.x, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, u.y, CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, make_int2(lo, hi));
}

// Sum over the LANES (8 or 16) consecutive lanes holding one head's row: swaps inside
// each quad (lane ^ 1, lane ^ 2), then the mirror of each 8-lane half (quad + other
// quad), then for 16 lanes the mirror of the row.
template <int LANES>
__device__ inline double row_sum(double v) {
  v += dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp<0x141>(v);  // row_half_mirror
  if (LANES == 16) v += dpp<0x140>(v);  // row_mirror
  return v;
}

// 1 / sqrt(s) for s > 0: the hardware estimate, then two Newton steps
// y <- y (3 - s y^2) / 2, each of which squares the relative error.
__device__ inline double rsqrt_refined(double s) {
  double y = __builtin_amdgcn_rsq(s);
  y = y * (1.5 - 0.5 * s * y * y);
  y = y * (1.5 - 0.5 * s * y * y);
  return y;
}

constexpr int kVecs = 64;    // 8-element vectors of the row per workgroup
constexpr int kPhases = 8;   // waves; wave p takes rows t0 + p, t0 + p + 8, ...

// grid: x = (block, group of 64 vectors of the row) with the group fastest, so that the
// workgroups that run side by side read neighbouring parts of the same rows (whole rows
// stream from each DRAM page), z = batch.  LANES = D / 8.  The
// element type is a template parameter, so the bf16 kernel holds only its own registers;
// rows are loaded U at a time and widened one at a time, as they are added.
template <int LANES, bool BF16>
__global__ __launch_bounds__(kVecs * kPhases) void sics_kernel(const uint8_t* __restrict__ x,
                                                               int64_t n, int block, int nb, int heads, int D,
                                                               int groups, double* __restrict__ out) {
  __shared__ double part[kPhases - 1][kVecs][8];
  const int blk = blockIdx.x / groups, grp = blockIdx.x - blk * groups;
  const int64_t b = blockIdx.z;
  const int hd = heads * D;
  const int l = threadIdx.x % kVecs, phase = threadIdx.x / kVecs;
  const int vec = grp * kVecs + l;
  const bool live = vec * 8 < hd;  // a head's lanes are live or dead together
  constexpr int esz = BF16 ? 2 : 4;
  const int64_t row_bytes = (int64_t)hd * esz;
  const int64_t t0 = (int64_t)blk * block, t1 = min(n, t0 + block);
  const uint8_t* p = x + (b * n + t0 + phase) * row_bytes + (int64_t)(live ? vec : 0) * 8 * esz;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto add_row = [&](const double* v) {
    double ss = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
    ss = row_sum<LANES>(ss);
    // branch-free (a zero row gets weight 0): the estimate is made for every lane and kept
    // opaque, so that the compiler does not turn the select into a branch per row, which
    // would defer the accumulation and keep every row's widened values live
    const bool nz = ss > 0;
    double r = rsqrt_refined(nz ? ss : 1.0);
    asm volatile("" : "+v"(r));
    const double inv = nz ? r : 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i] * inv;
  };
  // U rows in flight per lane: 4, so that a wave of even a 64-row block (8 rows) loads in two
  // batches and overlaps the second with the first's arithmetic (8 in flight: 66% of HBM on
  // 64-row blocks against 83%; 84% against 86% on 128-row blocks; 384-row blocks 74% either way)
  constexpr int U = 4;
  const uint4 zero = {0, 0, 0, 0};
  int64_t t = t0 + phase;
  for (; t + (U - 1) * kPhases < t1; t += U * kPhases) {
    uint4 a[U], c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a[u] = load_stream(p + u * kPhases * row_bytes);
      c[u] = BF16 ? zero : load_stream(p + u * kPhases * row_bytes + 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      double v[8];
      widen8<BF16>(a[u], c[u], v);
      add_row(v);
    }
    p += U * kPhases * row_bytes;
  }
  for (; t < t1; t += kPhases) {
    const uint4 a = load_stream(p);
    const uint4 c = BF16 ? zero : load_stream(p + 16);
    double v[8];
    widen8<BF16>(a, c, v);
    add_row(v);
    p += kPhases * row_bytes;
  }
  if (phase > 0)
#pragma unroll
    for (int i = 0; i < 8; ++i) part[phase - 1][l][i] = acc[i];
  __syncthreads();
  if (phase > 0) return;
  for (int q = 0; q < kPhases - 1; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += part[q][l][i];
  double sq = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) sq += acc[i] * acc[i];
  sq = row_sum<LANES>(sq);
  if (live && vec % LANES == 0) out[(b * heads + vec / LANES) * nb + blk] = sq;
}

}  // namespace

hipError_t launch_block_sics(const void* x, int bf16, int64_t batch, int heads, int D, int64_t n, int block,
                             double* scores, hipStream_t stream) {
  const int nb = (int)((n + block - 1) / block);
  const int vpr = heads * D / 8;  // 8-element vectors per row
  const int groups = (vpr + kVecs - 1) / kVecs;
  const dim3 grid((unsigned)(nb * groups), 1, (unsigned)batch);
  auto kern = D == 64 ? (bf16 ? sics_kernel<8, true> : sics_kernel<8, false>)
                      : (bf16 ? sics_kernel<16, true> : sics_kernel<16, false>);
  hipLaunchKernelGGL(kern, grid, dim3(kVecs * kPhases), 0, stream, (const uint8_t*)x, n, block, nb, heads, D,
                     groups, scores);
  return hipGetLastError();
}

}  // namespace vsa

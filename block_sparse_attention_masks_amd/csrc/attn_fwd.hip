// Block-sparse attention forward: exact softmax(Q K^T * scale) V over the key
// blocks a CSR mask keeps (SPADE summary, gist.science/ja/paper/2608.03335, "The
// solution" part 3: head-wise sparse attention on the kept blocks only; the
// pages' masks decide which blocks are kept).
//
// bf16 path (matrix cores).  A workgroup of NW waves owns 32 * NW query rows of
// one (batch, head, query block); each wave owns 32 of them, held in registers as
// the B operand of S^T = K Q^T.  NW is 12 or 8 when the query block is a multiple
// of 384 or 256 rows (one copy of each K/V tile then serves that many rows; the
// bytes copied per flop, not their latency, are what the copies cost), else 4;
// blocks of at most 64 rows split each tile's keys between two wave pairs, or,
// grouped, several consecutive blocks of at most 128 rows share a workgroup and walk
// the union of their kept key blocks (a wave computes only on its own block's).
// The kept key blocks are walked as one stream of 64-key tiles:
//   * tile t+1 is copied from HBM straight into the other half of a
//     double-buffered LDS stage (global_load_lds, 16 bytes per lane, no staging
//     registers) while tile t is computed; one wait + barrier per tile.  The walk
//     (32-bit scalar arithmetic) is advanced one tile ahead, after the products are
//     issued, to keep it off the loop head where every wave meets after the barrier.
//     Grouped walks of key blocks of <= 64 keys hold two tiles per stage (TW = 2),
//     one wait + barrier per pair: consecutive tiles then belong to different blocks,
//     and a wave whose block skips the first goes straight on to the second;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (M = keys, N = queries, K = head
//     dim): the accumulator gives each lane one query and 16 keys, so the row max
//     and row sum are in-lane plus one exchange between the half-waves;
//   * online softmax in the log2 domain with a lazy reference maximum: the
//     output is rescaled only when a row's maximum grows by more than 2^8, which
//     keeps every exponent <= 2^8 and leaves the normalised result unchanged;
//   * O^T += V^T P^T on the same instruction (M = head dim, N = queries, K =
//     keys), P rounded to bf16; the row sum adds the rounded values, so the
//     weights applied to V are exactly normalised.  Two V layouts (VT):
//       - VT: V was packed transposed, [batch, heads, 64-key tile, D, 64] (vt_pack_kernel,
//         one HBM pass), so a tile is one contiguous D x 64 block and a lane's 8 keys of one
//         head-dim row are 16 contiguous bytes: the A operand is a plain ds_read_b128.  The
//         K rows are read into the S product in a permuted order (bits 2 and 3 of the row
//         swapped) so that lane half g's P values are keys 8g..8g+7 of each 16-key group;
//       - else V stays row-major in LDS and ds_read_b64_tr_b16 delivers each lane its 8
//         keys of one head-dim column, in the order of the S accumulator layout (lane half
//         g holds keys 4g..4g+3 and 8+4g..8+4g+3).
//     Either way P feeds the product without any shuffle.  VT halves the LDS time of the V
//     reads (a 64-bit read moves half the bytes per cycle of a 128-bit one) and lets the
//     compiler schedule them, where the transposed reads need their wait in the same asm
//     block.  It needs a workspace for the packed copy and blocks of a multiple of 64 keys
//     (every tile then starts at a multiple of 64; tiled, the copy is in tile-major order).
// Ragged key tails are masked with -inf; query rows past the block or the
// sequence are computed but never stored.  A row with no kept block writes 0
// and lse = -inf.  Tiled (TL): q, k, v, o and lse are in raster order of a 3D grid
// whose tiles are the blocks; every row address goes through the tile-major
// permutation (see Tiling below) instead of the tensors being reordered.
//
// fp32 path: the same definition evaluated with fp32 FMA on the vector units,
// one thread per query row (used for small fp32 problems).
#include <math.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "group_union.h"
#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;      // query rows per 4-wave workgroup
constexpr int kBN = 64;       // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale slack (exponents stay <= 2^8)

// Work items to workgroups.  The dispatcher deals workgroup b to XCD b % 8.  chunk = 0: XCD x
// takes the contiguous range x per_xcd .. (x + 1) per_xcd - 1.  chunk = C (xcd_run): the items
// are cut into runs of 8 C and XCD x takes the x-th C of each run (the last, partial run keeps
// the dispatcher's order), so the 8 XCDs work on neighbouring items of one head, whose K and V
// they then share through the Infinity Cache, while each keeps C consecutive items for its L2.
struct Work {
  int64_t items, per_xcd;
  int nbq, mt_per_qb;
  int chunk = 0;
};

// Grouped query blocks: G consecutive query blocks of a slab share a workgroup of G * wpb
// waves and walk the union of their kept key blocks.  List u = slab * n_groups + group
// holds cnt[u] entries at col[u * cap ..], each with a mask of the rows that keep it.  The
// lists themselves are kernel arguments of their own (col in col_idx's place, mask, cnt),
// declared __restrict__ like the CSR: that is what lets the compiler read them with scalar
// loads.  Read through a struct's pointers they became vector loads, and the wait for such
// a load also waited for the next tile's copies just issued, so no copy overlapped compute.
struct Groups {
  int G, wpb, cap;
  int stride;  // group c stride + j holds query blocks c stride G + j + i stride, i < G
};

// Split key streams (SP): a row's kept-block list is cut into n contiguous chunks, each
// walked by its own workgroup, when there are too few rows to fill the chip.  A chunk
// writes its unnormalised fp32 output and (reference maximum in log2 units, row sum) for
// each of its rows (tiled: indexed by the raster row, the order of o and lse);
// split_merge_kernel adds the chunks in a fixed order.
struct Split {
  float* o;      // [n][rows][D]
  float* ml;     // [n][rows][2]
  int64_t rows;  // batch * heads * nq
  int n;
};

// Tokens in raster order of a T x H x W grid cut into tt x th x tw tiles, the attention
// blocks being the tiles in tile-major order (the order the tile reorder produces: STA,
// "Sliding tile attention", sec. 3): the rows are mapped on the fly instead of moved.
// NH, NW: tiles along H and W; P = th tw; V = tt P (tokens per tile); HW = H W.  A 64-row
// copy tile at within-tile offset r0 (a multiple of 64) sits at raster rows
// tile start + uni(r0) + lane(r) when the tile's h-w plane and the copy tile nest:
//   mode 1: P % 64 == 0 and tw | 64;  mode 2: P % 64 == 0 and 64 | tw;  mode 3: P | 64.
struct Tiling {
  int H, W, tt, th, tw, NH, NW, P, V, HW, mode;
  // n / d = (n m) >> (31 + l) for n < 2^31, with l = ceil(log2 d) and m = ceil(2^(31 + l) / d)
  // (the round-up reciprocal of Granlund and Montgomery): for d = NH NW and d = NW
  uint32_t m_plane, m_nw;
  int l_plane, l_nw;
  // uni(64 c) for the copy tiles c < ceil(V / 64) of a tile (V <= 64 kTiledMaxCopyTiles):
  // a table in the kernel arguments, so the walk reads one value per copy tile
  int uo_tab[kTiledMaxCopyTiles];
};

__device__ inline uint32_t div_magic(uint32_t n, uint32_t m, int l) {
  return (uint32_t)(((uint64_t)n * m) >> (31 + l));
}
// Raster row of the first token of tile `tile` (tile-major tile index).
__device__ inline int tile_start(const Tiling& t, int tile) {
  const uint32_t it_ = div_magic((uint32_t)tile, t.m_plane, t.l_plane);
  const uint32_t rem = (uint32_t)tile - it_ * (uint32_t)(t.NH * t.NW);
  const uint32_t ih = div_magic(rem, t.m_nw, t.l_nw), iw = rem - ih * (uint32_t)t.NW;
  return (int)(it_ * t.tt * t.HW + ih * t.th * t.W + iw * t.tw);
}

// Raster row (within one batch entry) of tile-major position p; every value is below
// the T H W tokens, which fit 31 bits.
__device__ inline int raster_row(const Tiling& t, int p) {
  const unsigned up = (unsigned)p, V = (unsigned)t.V, P = (unsigned)t.P, tw = (unsigned)t.tw;
  const unsigned tile = up / V, r = up - tile * V;
  const unsigned plane = (unsigned)(t.NH * t.NW), it_ = tile / plane, rem = tile - it_ * plane;
  const unsigned ih = rem / (unsigned)t.NW, iw = rem - ih * (unsigned)t.NW;
  const unsigned lt = r / P, rr = r - lt * P, lh = rr / tw, lw = rr - lh * tw;
  return (int)((it_ * t.tt + lt) * t.HW + (ih * t.th + lh) * t.W + iw * tw + lw);
}
// lane part for row r (0..63) of a full copy tile
__device__ inline int tile_lane(const Tiling& t, int r) {
  if (t.mode == 1) return (r / t.tw) * t.W + r % t.tw;
  if (t.mode == 2) return r;
  const int lt = r / t.P, rr = r - lt * t.P;
  return lt * t.HW + (rr / t.tw) * t.W + rr % t.tw;
}

// Stream of 64-key tiles over the kept blocks of one CSR row (wave-uniform).
// Key indices fit 31 bits with 64 to spare (the call checks nk), so the stream is walked
// in 32-bit scalar arithmetic.
struct TileIter {
  const int32_t* col;
  int e, e1;
  int k0, ke;
  int block_k;
  int nk;
  int ks = 0;  // first key of the current block
  // tiled: raster row of the block's first token, and the uniform raster offset of the
  // current copy tile within it
  int rb = 0, uo = 0;
  __device__ bool valid() const { return e < e1; }
  __device__ void open() {  // position on the first tile of block col[e]
    if (e < e1) {
      ks = col[e] * block_k;
      k0 = ks;
      ke = block_k < nk - ks ? ks + block_k : nk;
    }
  }
  __device__ void open(const Tiling& t) {
    open();
    if (e < e1) {
      rb = tile_start(t, col[e]);  // a block is a tile
      uo = 0;
    }
  }
  __device__ void next() {
    k0 += kBN;
    if (k0 >= ke) {
      ++e;
      open();
    }
  }
  __device__ void next(const Tiling& t) {
    k0 += kBN;
    if (k0 >= ke) {
      ++e;
      open(t);
      return;
    }
    // the next 64 rows of the same tile: one scalar read of the table
    uo = t.uo_tab[(k0 - ks) >> 6];
  }
};

// Value held by lane l ^ 32 (the other half-wave), via v_permlane32_swap (no LDS).
__device__ inline float xchg32(float x, int g) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(g == 0 ? r[1] : r[0]);
}

// ---- LDS layout --------------------------------------------------------------------
// K and V tiles are stored unpadded (row r of a 64-key tile at r * D elements), so a
// direct copy writes them, and the 16-byte chunks of each row are permuted by an XOR
// so the reads below are free of bank conflicts:
//   * K: chunk c of row r sits at slot c ^ swz_k(r).  A K-fragment read touches 32
//     consecutive rows at one chunk pair; D = 128 spreads 16 rows over all 16 slots,
//     D = 64 (8 slots, two rows per 256 bytes) spreads row pairs over 8 slots.
//   * V: chunk c of row r sits at slot c ^ swz_v(r).  A transposed read touches 4
//     consecutive rows x 64 bytes; the shift moves each of the 4 rows to its own
//     quarter of the banks.
template <int D> __device__ inline int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D> __device__ inline int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
//   * V^T (VT): row d of the tile (its 64 keys, 128 bytes, 8 chunks) at d * 64 elements,
//     chunk c at slot c ^ swz_vt(d).  A V-fragment read touches 32 consecutive rows at one
//     chunk; any 16 consecutive rows, 8 of each parity, land on distinct banks.
__device__ inline int swz_vt(int r) { return (r >> 1) & 7; }
// VT: key row of the tile that A-operand row c (0..31) of the S product reads: bits 2 and 3
// of c swapped.  The accumulator then holds, in lane half g, keys 16 j + 8 g + (a & 7) for
// element a of the 16, j = a >> 3 (without it: 8 (a >> 2) + 4 g + (a & 3)).
__device__ inline int kperm(int c) { return (c & ~12) | ((c & 4) << 1) | ((c & 8) >> 1); }

// s_waitcnt vmcnt(N), leaving the other counters alone (gfx9 encoding: vmcnt low
// bits [3:0] and high bits [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N> __device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One wave copies 64 x 16 bytes from global memory to LDS: lane i's 16 bytes land at
// lds + 16 * i (lds is wave-uniform).
__device__ inline void load_lds16(const uint16_t* src, uint16_t* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

typedef unsigned long long u64_t;

// V fragments of one 16-key group for every 32-column slice of the head dim:
// vf[t][i] = V[key_i][32 t + lane % 32] with key_i = 4 g + i (i < 4) and 8 + 4 g + i - 4
// (i >= 4), g = lane / 32.  The reads and their wait sit in one asm block: the compiler
// would otherwise wait for every outstanding global->LDS copy before a transposed read.
template <int D>
__device__ inline void read_v_step(bf16x8 (&vf)[D / 32], uint32_t base, const int (&voff)[D / 32]);

template <>
__device__ inline void read_v_step<128>(bf16x8 (&vf)[4], uint32_t base, const int (&voff)[4]) {
  u64_t r0, r1, r2, r3, r4, r5, r6, r7;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n"
      "ds_read_b64_tr_b16 %1, %8 offset:2048\n"
      "ds_read_b64_tr_b16 %2, %9\n"
      "ds_read_b64_tr_b16 %3, %9 offset:2048\n"
      "ds_read_b64_tr_b16 %4, %10\n"
      "ds_read_b64_tr_b16 %5, %10 offset:2048\n"
      "ds_read_b64_tr_b16 %6, %11\n"
      "ds_read_b64_tr_b16 %7, %11 offset:2048\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(base + 2 * voff[0]), "v"(base + 2 * voff[1]), "v"(base + 2 * voff[2]),
        "v"(base + 2 * voff[3])
      : "memory");
  const u64_t r[8] = {r0, r1, r2, r3, r4, r5, r6, r7};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const u64_t pr[2] = {r[2 * t], r[2 * t + 1]};
    vf[t] = __builtin_bit_cast(bf16x8, pr);
  }
}

template <>
__device__ inline void read_v_step<64>(bf16x8 (&vf)[2], uint32_t base, const int (&voff)[2]) {
  u64_t r0, r1, r2, r3;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n"
      "ds_read_b64_tr_b16 %1, %4 offset:1024\n"
      "ds_read_b64_tr_b16 %2, %5\n"
      "ds_read_b64_tr_b16 %3, %5 offset:1024\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(base + 2 * voff[0]), "v"(base + 2 * voff[1])
      : "memory");
  const u64_t r[4] = {r0, r1, r2, r3};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const u64_t pr[2] = {r[2 * t], r[2 * t + 1]};
    vf[t] = __builtin_bit_cast(bf16x8, pr);
  }
}

// The two tiles after the next one, kept when a stage holds two tiles.
template <int TW>
struct Lookahead {
  TileIter n2, n3;
};
template <>
struct Lookahead<1> {};

// LDS copy slots: two stages of TW stream tiles each.
template <int D, int TW>
struct Smem {
  uint16_t k[2 * TW][kBN * D];
  uint16_t v[2 * TW][kBN * D];
};

template <int D, int KS, int NW, bool GR, bool TL, int TW, bool SP, bool VT>
__global__ __launch_bounds__(NW * kWave, NW == 4 ? 2 : 1) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    int64_t nq, int64_t nk, int heads, int block_q, int block_k,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const int32_t* __restrict__ gmask, const int32_t* __restrict__ gcnt, int n_slabs,
    float scale_log2, Work wk, Groups gp, Tiling tg, Split sp) {
  __shared__ __attribute__((aligned(1024))) Smem<D, TW> sm;
  // TW = 2: two stream tiles per stage, so per wait and barrier.  That pays off for grouped
  // blocks of 64 rows, where consecutive tiles belong to different key blocks and so often
  // to different waves: a wave with nothing to do for the first tile goes on to the second
  // instead of waiting at a barrier.
  static_assert(TW == 1 || (GR && NW >= 8 && !TL), "two tiles per stage: grouped, untiled, 8 or 12 waves");
  static_assert(KS == 1 || NW == 4, "key split runs with 4 waves");
  static_assert(!GR || KS == 1, "grouped query blocks use whole tiles");
  constexpr int BM = 32 * NW / KS;
  constexpr int NST = 2 / KS;
  constexpr int SPR = D / 8;              // 16-byte slots per row
  constexpr int RPC = 64 / SPR;           // rows per 1 KB wave-load
  constexpr int CB = kBN / RPC;           // wave-loads per tensor per tile
  constexpr int NJ = (2 * CB + NW - 1) / NW;  // wave-loads per wave per tile (K and V together)

  // work item: (batch, head, query block, row tile) -- or, grouped, (batch, head, group
  // of gp.G query blocks); wk.nbq counts query blocks or groups
  const int64_t bid = blockIdx.x;
  int64_t item;
  if (wk.chunk == 0) {
    item = (bid % 8) * wk.per_xcd + bid / 8;
  } else {
    const int64_t c8 = 8 * (int64_t)wk.chunk, full = wk.items / c8 * c8;
    item = bid < full ? bid / c8 * c8 + (bid % 8) * wk.chunk + bid / 8 % wk.chunk : bid;
  }
  if (item >= wk.items) return;
  int chunk = 0;  // SP: the chunk of the row's key stream, innermost
  if constexpr (SP) {
    chunk = (int)(item % sp.n);
    item /= sp.n;
  }
  const int mt = (int)(item % wk.mt_per_qb);
  int64_t rest = item / wk.mt_per_qb;
  const int qb = (int)(rest % wk.nbq);
  rest /= wk.nbq;
  const int h = (int)(rest % heads);
  const int64_t b = rest / heads;

  const int tid = threadIdx.x, l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = l & 31, g = l >> 5;
  const int qw = KS == 1 ? w : (w & 1);
  const int kh = KS == 1 ? 0 : (w >> 1);
  const int row_stride = heads * D;
  // this wave's 32 query rows [q_w, q_hi)
  int64_t q_w, q_hi;
  int lq = 0;  // grouped: the wave's query block within the group
  if constexpr (GR) {
    lq = w / gp.wpb;
    const int64_t qbw = (int64_t)(qb / gp.stride) * gp.stride * gp.G + qb % gp.stride + (int64_t)lq * gp.stride;
    q_w = qbw * block_q + (int64_t)(w % gp.wpb) * 32;
    q_hi = lq < gp.G ? min(min((qbw + 1) * block_q, nq), q_w + 32) : q_w;
  } else {
    const int64_t q_lo = (int64_t)qb * block_q + (int64_t)mt * BM;
    if (q_lo >= min((int64_t)(qb + 1) * block_q, nq)) return;
    q_w = q_lo + qw * 32;
    q_hi = min(min((int64_t)(qb + 1) * block_q, nq), q_lo + BM);
  }

  const int64_t slab = n_slabs == 1 ? 0 : b * heads + h;
  TileIter it;
  if constexpr (GR) {  // the union of the group's kept blocks, with a row-membership mask
    const int64_t u = slab * wk.nbq + qb;
    it = TileIter{col_idx, (int)(u * gp.cap), (int)(u * gp.cap) + gcnt[u], 0, 0, block_k, (int)nk};
  } else {
    const int64_t r = slab * wk.nbq + qb;
    it = TileIter{col_idx, row_ptr[r], row_ptr[r + 1], 0, 0, block_k, (int)nk};
  }
  if constexpr (SP) {  // this chunk's share of the entries, split as evenly as integers allow
    const int e0 = it.e, ne = it.e1 - it.e;
    it.e = e0 + (int)((int64_t)ne * chunk / sp.n);
    it.e1 = e0 + (int)((int64_t)ne * (chunk + 1) / sp.n);
  }
  if constexpr (TL) it.open(tg);
  else it.open();
  const uint16_t* kbase = k + (b * nk * heads + h) * (int64_t)D;
  // VT: v is the packed V^T, one D x 64 block per (batch, head, 64-key tile)
  const uint16_t* vbase = VT ? v + (b * heads + h) * ((nk + kBN - 1) / kBN) * (int64_t)(D * kBN)
                             : v + (b * nk * heads + h) * (int64_t)D;

  // Copy plan: wave-load c = w + NW j (c < 2 CB) moves RPC rows of K (c < CB) or of V
  // (chunk-block c - CB) of the tile; the tile base is wave-uniform, each lane adds a
  // loop-invariant row and chunk.  Rows past the last key repeat it (masked later).
  const uint32_t row_bytes = 2u * (uint32_t)row_stride;
  // VT: a V wave-load c - CB moves head-dim rows 8 (c - CB) .. + 7 of the tile's D x 64
  // block (8 chunks of 16 bytes each); ch16 is then the lane's whole byte offset in the block
  int lrow[NJ];
  uint32_t ch16[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = w + NW * j;
    const int cb = c < CB ? c : c - CB;
    if (VT && c >= CB) {
      const int d = cb * 8 + l / 8;
      lrow[j] = 0;
      ch16[j] = 128u * d + 16u * ((l % 8) ^ swz_vt(d));
    } else {
      lrow[j] = cb * RPC + l / SPR;
      ch16[j] = 16u * ((l % SPR) ^ (c < CB ? swz_k<D>(lrow[j]) : swz_v<D>(lrow[j])));
    }
  }
  int loff[NJ];  // tiled: lane part of row lrow[j] of a full copy tile
#pragma unroll
  for (int j = 0; j < NJ; ++j) loff[j] = TL ? tile_lane(tg, lrow[j]) : 0;
  auto issue = [&](const TileIter& t_, int stage) {
    const int k0 = t_.k0, ke = t_.ke;
    const int last = min(ke - k0, kBN) - 1;
    if constexpr (TL) {
      // rows of a copy tile: tile start + uniform part + lane part.  The lane part holds for
      // every row the tile has, so a partial copy tile (the tail of a tile that is not a
      // multiple of 64 tokens) takes it too; its rows past the last read the first row
      // (finite values, masked out later)
      // the copy tile's first row is a scalar; the lane part is a 32-bit byte offset (the
      // call checks that a copy tile's rows lie within 2^32 bytes and 2^24 rows of it)
      const int64_t r0 = t_.rb + t_.uo;
      const char* kt = (const char*)(kbase + r0 * row_stride);
      // VT: the packed copy is in tile-major key order, so the tile is k0 / 64 as untiled
      const char* vt = VT ? (const char*)(vbase + (int64_t)(k0 / kBN) * (D * kBN))
                          : (const char*)(vbase + r0 * row_stride);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = w + NW * j;
        if (c < 2 * CB) {
          const uint32_t ro = VT && c >= CB ? ch16[j]
                                            : __umul24((uint32_t)(lrow[j] <= last ? loff[j] : 0), row_bytes) + ch16[j];
          if (c < CB)
            load_lds16((const uint16_t*)(kt + ro), sm.k[stage] + c * 512);
          else
            load_lds16((const uint16_t*)(vt + ro), sm.v[stage] + (c - CB) * 512);
        }
      }
    } else {
      const char* kt = (const char*)(kbase + (int64_t)k0 * row_stride);
      // VT: k0 is a multiple of 64; keys past nk are zeros of the packed copy
      const char* vt = VT ? (const char*)(vbase + (int64_t)(k0 / kBN) * (D * kBN))
                          : (const char*)(vbase + (int64_t)k0 * row_stride);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = w + NW * j;
        if (c < 2 * CB) {
          const uint32_t ro = VT && c >= CB ? ch16[j] : __umul24((uint32_t)min(lrow[j], last), row_bytes) + ch16[j];
          if (c < CB)
            load_lds16((const uint16_t*)(kt + ro), sm.k[stage] + c * 512);
          else
            load_lds16((const uint16_t*)(vt + ro), sm.v[stage] + (c - CB) * 512);
        }
      }
    }
  };

  const int64_t my_q = q_w + col;
  // row of this lane's query in q, o and lse (tiled: its raster row)
  const int64_t my_row = TL && my_q < q_hi ? (int64_t)raster_row(tg, (int)my_q) : my_q;
  bf16x8 qf[D / 16];
  {
    const bool ok = my_q < q_hi;
    const uint16_t* qp = q + ((b * nq + (ok ? my_row : 0)) * heads + h) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 u = ok ? *(const u32x4*)(qp + 16 * s) : u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, u);
    }
  }
  if (it.valid()) issue(it, 0);
  if constexpr (TW == 2) {
    TileIter t1 = it;
    t1.next();
    if (t1.valid()) issue(t1, 1);
  }

  f32x16 acc_o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int a = 0; a < 16; ++a) acc_o[t][a] = 0.f;
  float m_ref = -INFINITY, l_run = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  // the K row this lane's A-operand row reads (VT: permuted), and its slot:
  // K slot of (row 32 st + krow, chunk 2 kd + g) = (2 kd) ^ kx
  const int krow = VT ? kperm(col) : col;
  const int kx = g ^ swz_k<D>(krow);
  // VT: V slot of (head-dim row 32 t + col, chunk 4 kh + 2 kk + g) = (2 kk) ^ vxg
  const int vxg = (4 * kh) ^ g ^ swz_vt(col);
  const int jv = (l & 15) >> 2, c4 = l & 3, m2 = (l >> 4) & 1;
  int voff[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
    voff[t] = (4 * g + jv) * D + 8 * (((4 * t + 2 * m2 + (c4 >> 1)) ^ swz_v<D>(4 * g + jv))) + 4 * (c4 & 1);
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();

  // nx (the tile after it) is advanced one iteration ahead, after the products are issued,
  // so the scalar work of the walk is not queued on the scalar unit by every wave at once
  // at the top of the loop, where it would delay the copies and the first products
  auto advance = [&](TileIter& t_) {
    if constexpr (TL) t_.next(tg);
    else t_.next();
  };
  // TW = 2: tiles n2 and n3 follow nx; slots cycle 0..3, a stage holding slots (0, 1) or
  // (2, 3), and the first tile of a stage copies the next two into the other stage
  TileIter nx = it;
  advance(nx);
  [[maybe_unused]] Lookahead<TW> la;
  if constexpr (TW == 2) {
    la.n2 = nx;
    la.n2.next();
    la.n3 = la.n2;
    la.n3.next();
  }
  int buf = 0;
  while (it.valid()) {
    const int valid = min(kBN, it.ke - it.k0);
    if constexpr (TW == 1) {
      if (nx.valid()) issue(nx, buf ^ 1);
    } else if ((buf & 1) == 0) {
      if (la.n2.valid()) issue(la.n2, buf ^ 2);
      if (la.n3.valid()) issue(la.n3, buf ^ 3);
    }
    const uint16_t* sk = sm.k[buf];
    const uint16_t* sv = sm.v[buf];
    // grouped: a wave whose query block does not keep this key block only helps copy it
    if (!GR || ((gmask[it.e] >> lq) & 1)) {
    f32x16 s[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int a = 0; a < 16; ++a) s[st][a] = 0.f;
    bf16x8 kf[D / 16][NST];  // the whole K tile of this wave, read before the first product
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd)
#pragma unroll
      for (int st = 0; st < NST; ++st)
        kf[kd][st] = *(const bf16x8*)(sk + (32 * (kh + st) + krow) * D + 8 * ((2 * kd) ^ kx));
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd)
#pragma unroll
      for (int st = 0; st < NST; ++st)
        s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kd][st], qf[kd], s[st], 0, 0, 0);
    if (valid < kBN) {
      asm volatile("" ::: "memory");
      const int lim = valid - (VT ? 8 : 4) * g - 32 * kh;  // key index minus its lane part
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int a = 0; a < 16; ++a)
          if (32 * st + (VT ? 16 * (a >> 3) + (a & 7) : 8 * (a >> 2) + (a & 3)) >= lim) s[st][a] = -INFINITY;
    }
    float mx = s[0][0];
    if constexpr (NST == 2) {
#pragma unroll
      for (int a = 0; a < 16; ++a) mx = fmaxf(fmaxf(mx, s[0][a]), s[1][a]);
    } else {
#pragma unroll
      for (int a = 1; a < 15; a += 2) mx = fmaxf(fmaxf(mx, s[0][a]), s[0][a + 1]);
      mx = fmaxf(mx, s[0][15]);
    }
    mx = fmaxf(mx, xchg32(mx, g)) * scale_log2;
    const bool grow = mx > m_ref + kRescaleLog2;
    if (__ballot(grow)) {
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
    const float m_use = KS == 1 ? m_ref : (m_ref == -INFINITY ? 0.f : m_ref);
    bf16x8 pf[2 * NST];
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int a = 0; a < 16; ++a)
        pf[2 * st + (a >> 3)][a & 7] =
            (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[st][a], scale_log2, -m_use));
    float psum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2 * NST; ++kk) {
      const bf16x2* pp = (const bf16x2*)&pf[kk];
#pragma unroll
      for (int i = 0; i < 4; ++i) psum = __builtin_amdgcn_fdot2_f32_bf16(pp[i], ones, psum, false);
    }
    l_run += psum;
#pragma unroll
    for (int kk = 0; kk < 2 * NST; ++kk) {
      bf16x8 vf[D / 32];
      if constexpr (VT) {
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
          vf[t] = *(const bf16x8*)(sv + (32 * t + col) * kBN + 8 * ((2 * kk) ^ vxg));
      } else {
        read_v_step<D>(vf, lds_addr(sv + 16 * (2 * kh + kk) * D), voff);
      }
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
        acc_o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t], pf[kk], acc_o[t], 0, 0, 0);
    }
    }
    if constexpr (TW == 1) {
      TileIter nn = nx;
      advance(nn);
      wait_vmcnt<0>();               // the next tile's loads have landed
      __builtin_amdgcn_s_barrier();  // ... for everyone; this tile is no longer read
      buf ^= 1;
      it = nx;
      nx = nn;
    } else {
      TileIter nn = la.n3;
      nn.next();
      if (buf & 1) {
        wait_vmcnt<0>();               // the next stage's loads have landed
        __builtin_amdgcn_s_barrier();  // ... for everyone; this stage is no longer read
      }
      buf = (buf + 1) & 3;
      it = nx;
      nx = la.n2;
      la.n2 = la.n3;
      la.n3 = nn;
    }
  }

  // ---- epilogue
  if constexpr (KS == 2) {
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
  const float l_tot = l_run + xchg32(l_run, g);
  if constexpr (SP) {  // the chunk's unnormalised output, its reference maximum and row sum
    if (my_q < q_hi) {
      const int64_t row = (int64_t)chunk * sp.rows + (b * heads + h) * nq + my_row;  // tiled: raster row
      float* op = sp.o + row * D;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          float4 ov;
          ov.x = acc_o[t][4 * a4];
          ov.y = acc_o[t][4 * a4 + 1];
          ov.z = acc_o[t][4 * a4 + 2];
          ov.w = acc_o[t][4 * a4 + 3];
          *(float4*)(op + 32 * t + 8 * a4 + 4 * g) = ov;
        }
      if (g == 0) *(float2*)(sp.ml + 2 * row) = float2{m_ref, l_tot};
    }
    return;
  }
  if (my_q < q_hi) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = o + ((b * nq + my_row) * heads + h) * D;
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
      lse[(b * heads + h) * nq + my_row] =
          l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * 0.6931471805599453f : -INFINITY;
  }
}

// V^T packing for the VT forward: v [batch, nk, heads, D] -> vt [batch, heads, ceil(nk / 64),
// D, 64], keys past nk zero; tiled (TL), key p of the packed order is raster row
// raster_row(p), so the copy is in tile-major order.  Workgroup = one (batch, 64-key tile) and
// every gridDim.y-th pair (D = 128) or quad (D = 64) of heads -- all heads, streaming whole token
// rows, unless there are too few (batch, tile) workgroups to fill the chip; thread = 8 keys x 8
// head-dim columns of one head (16-byte loads of 8 key rows, an 8 x 8 transpose in registers,
// 16-byte stores of 8 head-dim rows), kPackThreads / D heads at a time.  One HBM read and one
// write of V.
constexpr int kPackThreads = 256;
template <int D, bool TL>
__global__ __launch_bounds__(kPackThreads) void vt_pack_kernel(const uint16_t* __restrict__ v,
                                                               uint16_t* __restrict__ vt, int64_t nk, int heads,
                                                               int64_t ntile, Tiling tg) {
  constexpr int DC = D / 8;                // 8-column chunks of a row
  constexpr int HP = kPackThreads / D;     // heads per pass
  const int64_t tile = blockIdx.x % ntile, b = blockIdx.x / ntile;
  const int t = threadIdx.x % D, hsub = threadIdx.x / D;
  const int dc = t % DC, kg = t / DC;
  // tiled: the 8 keys start at a multiple of 8, so when tw is a multiple of 8 they are 8
  // consecutive tokens of one raster row of the tile, and one raster_row serves all of them
  const int64_t key0 = tile * kBN + kg * 8;
  const bool run8 = TL && tg.tw % 8 == 0;
  const int64_t row0 = run8 && key0 < nk ? (int64_t)raster_row(tg, (int)key0) : key0;
  int64_t row[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t key = key0 + j;
    row[j] = !TL ? key : (run8 ? row0 + j : (key < nk ? (int64_t)raster_row(tg, (int)key) : key));
  }
  for (int h = (int)blockIdx.y * HP + hsub; h < heads; h += HP * (int)gridDim.y) {
    u32x4 in[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      in[j] = key0 + j < nk ? *(const u32x4*)(v + ((b * nk + row[j]) * heads + h) * D + dc * 8)
                            : u32x4{0, 0, 0, 0};
    uint16_t* out = vt + ((b * heads + h) * ntile + tile) * (int64_t)(D * kBN) + (int64_t)(dc * 8) * kBN + kg * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // head-dim row dc 8 + i: keys kg 8 .. kg 8 + 7
      u32x4 r;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const uint32_t lo = in[2 * q2][i / 2], hi = in[2 * q2 + 1][i / 2];
        r[q2] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      *(u32x4*)(out + (int64_t)i * kBN) = r;
    }
  }
}

// Merge of split key streams: thread = 4 output elements of one (batch, head, query) row.
// With m the largest of the chunks' reference maxima, chunk c counts with weight
// 2^(m_c - m); the chunks are added in order c = 0, 1, ..., so the result is deterministic.
template <int D>
__global__ __launch_bounds__(256) void split_merge_kernel(const float* __restrict__ opart,
                                                          const float* __restrict__ ml, int n, int64_t rows,
                                                          int heads, int64_t nq, uint16_t* __restrict__ o,
                                                          float* __restrict__ lse) {
  constexpr int C = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= rows * C) return;
  const int64_t row = gid / C;
  const int d0 = (int)(gid % C) * 4;
  float m = -INFINITY;
  for (int c = 0; c < n; ++c) m = fmaxf(m, ml[2 * (c * rows + row)]);
  float l = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (m != -INFINITY) {
    for (int c = 0; c < n; ++c) {
      const float2 mc = *(const float2*)(ml + 2 * (c * rows + row));
      const float a = __builtin_amdgcn_exp2f(mc.x - m);
      l += a * mc.y;
      const float4 x = *(const float4*)(opart + (c * rows + row) * D + d0);
      acc[0] += a * x.x;
      acc[1] += a * x.y;
      acc[2] += a * x.z;
      acc[3] += a * x.w;
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t q = row % nq, bh = row / nq, h = bh % heads, b = bh / heads;
  bf16x4 ov;
#pragma unroll
  for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(acc[i] * inv);
  *(bf16x4*)(o + ((b * nq + q) * heads + h) * D + d0) = ov;
  if (lse != nullptr && d0 == 0)
    lse[row] = l > 0.f ? (m + __builtin_amdgcn_logf(l)) * 0.6931471805599453f : -INFINITY;
}

// fp32: one thread per (batch, head, query); plain online softmax over the kept keys.
template <int D, bool TL>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int64_t batch, int64_t nq, int64_t nk,
    int heads, int block_q, int block_k, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, int n_slabs, int nbq, float scale, Tiling tg) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= batch * heads * nq) return;
  const int64_t tq = gid % nq;
  const int h = (int)((gid / nq) % heads);
  const int64_t b = gid / (nq * heads);
  const int64_t stride = (int64_t)heads * D;
  float qv[D], acc[D];
  const int64_t qrow = TL ? (int64_t)raster_row(tg, (int)tq) : tq;  // row in q, o and lse
  const float* qp = q + (b * nq + qrow) * stride + (int64_t)h * D;
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
      const int64_t krow = TL ? (int64_t)raster_row(tg, (int)kt) : kt;
      const float* kp = k + (b * nk + krow) * stride + (int64_t)h * D;
      const float* vp = v + (b * nk + krow) * stride + (int64_t)h * D;
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
  float* op = o + (b * nq + qrow) * stride + (int64_t)h * D;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
  if (lse != nullptr) lse[(b * heads + h) * nq + qrow] = lsum > 0.f ? m + logf(lsum) : -INFINITY;
}

}  // namespace

namespace {

// How a call runs: grouped (wpb waves per query block, G blocks per workgroup of nw
// waves), or per query block (ks = 2 key split for blocks <= 64 rows, else nw waves).
struct FwdPlan {
  bool grouped;
  int ks, nw, G, wpb, n_groups;
  size_t ws_bytes;
  int tw = 1;      // stream tiles per LDS stage
  int splits = 1;  // chunks per row's key stream (split_merge_kernel adds them)
  bool vt = false;     // V packed transposed (vt_pack_kernel) into the workspace at vt_off
  size_t vt_off = 0;
};

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workgroups the chip runs at once for a given width (one 8- or 12-wave workgroup per CU,
// or two 4-wave ones: the LDS stages take 64 KB each).
constexpr int kCUs = 256;
inline int64_t wg_slots(int nw) { return (int64_t)kCUs * (nw == 4 ? 2 : 1); }

// Split each row's key stream when the rows alone cannot fill one round of workgroups on
// the chip: enough chunks for about kSplitRounds rounds, at most 8, and on average at least
// 8 key blocks per chunk (the kept-list lengths are only known on the device; n_kblocks
// bounds them).  Returns the bytes of the partial outputs, n * rows * (D + 2) fp32, or 0
// when the problem is not split.  (Between one and two rounds, splitting was measured to
// gain nothing: 888 rows of 115 64-key tiles ran 0.473 ms unsplit and 0.475 ms in two
// chunks; such a problem is bound by the bytes copied per flop, not by occupancy.)
constexpr int kSplitRounds = 2;
size_t plan_split(const AttnArgs& a, FwdPlan& p, int64_t items) {
  const int64_t slots = wg_slots(p.nw);
  const int64_t nbk = (a.nk + a.block_k - 1) / a.block_k;
  p.splits = 1;
  if (items >= slots || nbk < 16) return 0;
  int64_t n = (kSplitRounds * slots + items - 1) / items;
  n = std::min<int64_t>(n, std::min<int64_t>(8, nbk / 8));
  if (n < 2) return 0;
  const int64_t rows = a.batch * a.heads * a.nq;
  p.splits = (int)n;
  return align256(4 * (size_t)(n * rows * a.head_dim)) + align256(8 * (size_t)(n * rows));
}

// Groups of G query blocks `stride` apart over nbq blocks: whole runs of stride * G blocks,
// each giving `stride` groups (the last run's groups may be partly or wholly past nbq).
int64_t group_count(int64_t nbq, int G, int stride) {
  return (nbq + (int64_t)stride * G - 1) / ((int64_t)stride * G) * stride;
}

// Workspace bytes of the union lists of a grouped plan: entries, row masks, counts.
size_t union_bytes(int64_t lists, int64_t nbk) {
  return 2 * align256(4 * (size_t)(lists * nbk)) + align256(4 * (size_t)lists);
}

FwdPlan plan_fwd(const AttnArgs& a, bool have_ws) {
  FwdPlan p{false, 1, 4, 1, 1, 0, 0};
  const int64_t nbq = (a.nq + a.block_q - 1) / a.block_q, nbk = (a.nk + a.block_k - 1) / a.block_k;
  const int wpb = (a.block_q + 31) / 32;
  // query blocks of <= 128 rows: group them when enough workgroups remain to fill the chip
  if (wpb <= 4) {
    for (int nw : {12, 8, 4}) {
      if (nw % wpb) continue;
      const int G = nw / wpb;
      const int64_t n_groups = group_count(nbq, G, a.group_stride);
      const int64_t items = a.batch * a.heads * n_groups;
      const int64_t lists = (int64_t)a.n_slabs * n_groups;
      if (G < 2 || items < (nw == 4 ? 512 : 256) || lists * nbk > 0x7fffffff) continue;
      p = FwdPlan{true, 1, nw, G, wpb, (int)n_groups, union_bytes(lists, nbk)};
      break;
    }
  }
  if (p.grouped && have_ws) {
    // every tile its own block (see the kernel); the tiled kernels have no registers to spare
    if (p.nw >= 8 && a.block_k <= kBN && !a.tiled) p.tw = 2;
    return p;
  }
  const size_t want_ws = p.grouped ? p.ws_bytes : 0;
  p = FwdPlan{false, a.block_q <= kBM / 2 ? 2 : 1, 4, 1, 1, 0, 0};
  if (p.ks == 1) p.nw = a.block_q % 384 == 0 ? 12 : (a.block_q % 256 == 0 ? 8 : 4);
  const int bm = 32 * p.nw / p.ks;
  const size_t part = plan_split(a, p, a.batch * a.heads * nbq * ((a.block_q + bm - 1) / bm));
  if (!have_ws) p.splits = 1;  // without a workspace: one workgroup per row
  p.ws_bytes = std::max(part, want_ws);
  return p;
}

// Bytes of the packed V^T when a call can use it, else 0: key blocks of a multiple of 64
// (tiles start at multiples of 64, in tile-major order when tiled), and at least as many
// queries as keys, so that each key tile is read by many query blocks and one packing pass
// over V pays off.
size_t vt_bytes(const AttnArgs& a) {
  if (a.block_k % kBN != 0 || a.nq < a.nk) return 0;
  // the packing kernel's grid: one workgroup per (batch, tile), at most 2^31 - 1
  if (a.batch * ((a.nk + kBN - 1) / kBN) > (int64_t)INT32_MAX) return 0;
  return align256(2 * (size_t)(a.batch * a.heads) * (size_t)((a.nk + kBN - 1) / kBN) * kBN * (size_t)a.head_dim);
}

// The plan for `have` workspace bytes: the grouped / split plan when its lists and partials
// fit, then the packed V^T after them when it fits too.
FwdPlan plan_fwd_ws(const AttnArgs& a, size_t have) {
  const bool core = have >= plan_fwd(a, true).ws_bytes;
  FwdPlan p = plan_fwd(a, core);
  if (!core) p.ws_bytes = 0;  // neither grouped nor split: no bytes of the workspace used yet
  const size_t vb = vt_bytes(a);
  if (vb && have >= p.ws_bytes && have - p.ws_bytes >= vb) {
    p.vt = true;
    p.vt_off = p.ws_bytes;
    p.ws_bytes += vb;
  }
  return p;
}

// Kernel view of the tile grid (a.tiled) and its copy mode; all zero when not tiled.
Tiling make_tiling(const AttnArgs& a) {
  Tiling t{};
  if (!a.tiled) return t;
  t.H = a.H;
  t.W = a.W;
  t.tt = a.tt;
  t.th = a.th;
  t.tw = a.tw;
  t.NH = a.H / a.th;
  t.NW = a.W / a.tw;
  t.P = a.th * a.tw;
  t.V = a.tt * t.P;
  t.HW = a.H * a.W;
  t.mode = tiling_mode(a.th, a.tw);
  // uni(r0) of copy tile r0 = 64 c: the raster offset of tile position r0 (its lane part
  // is added per lane; in every supported mode the two add up for all 64 rows)
  for (int c = 0; c < kTiledMaxCopyTiles; ++c) {
    const int r = kBN * c;
    if (r >= t.V) {
      t.uo_tab[c] = 0;
      continue;
    }
    const int lt = r / t.P, rr = r % t.P;
    t.uo_tab[c] = lt * t.HW + (rr / t.tw) * t.W + rr % t.tw;
  }
  auto magic = [](uint32_t d, uint32_t& m, int& l) {
    l = 0;
    while ((1ull << l) < d) ++l;
    m = (uint32_t)(((1ull << (31 + l)) + d - 1) / d);
  };
  magic((uint32_t)(t.NH * t.NW), t.m_plane, t.l_plane);
  magic((uint32_t)t.NW, t.m_nw, t.l_nw);
  return t;
}

}  // namespace

int64_t tiling_lane_span(int H, int W, int th, int tw) {
  const int P = th * tw;
  switch (tiling_mode(th, tw)) {
    case 1: return (int64_t)(kBN / tw - 1) * W + tw - 1;
    case 2: return kBN - 1;
    case 3: return (int64_t)(kBN / P - 1) * H * W + (int64_t)(th - 1) * W + tw - 1;
    default: return -1;
  }
}

int tiling_mode(int th, int tw) {
  const int P = th * tw;
  if (P % kBN == 0 && kBN % tw == 0) return 1;
  if (P % kBN == 0 && tw % kBN == 0) return 2;
  if (kBN % P == 0) return 3;
  return 0;
}

size_t attn_fwd_workspace(const AttnArgs& a) { return plan_fwd_ws(a, SIZE_MAX).ws_bytes; }
size_t attn_fwd_workspace_min(const AttnArgs& a) { return plan_fwd(a, true).ws_bytes; }

hipError_t launch_attn_fwd(const AttnArgs& a, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int nbq = (int)((a.nq + a.block_q - 1) / a.block_q);
  const Tiling tg = make_tiling(a);
  if (a.dtype == 0) {
    const int64_t n = a.batch * a.heads * a.nq;
    const dim3 grid((unsigned)((n + 255) / 256));
    auto launch32 = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, (const float*)a.q, (const float*)a.k,
                         (const float*)a.v, (float*)a.o, a.lse, a.batch, a.nq, a.nk, a.heads, a.block_q,
                         a.block_k, a.row_ptr, a.col_idx, a.n_slabs, nbq, a.scale, tg);
    };
    if (a.head_dim == 64) {
      if (a.tiled) launch32(attn_fwd_f32_kernel<64, true>);
      else launch32(attn_fwd_f32_kernel<64, false>);
    } else {
      if (a.tiled) launch32(attn_fwd_f32_kernel<128, true>);
      else launch32(attn_fwd_f32_kernel<128, false>);
    }
    return hipGetLastError();
  }
  const float sl2 = a.scale * kLog2e;
  const FwdPlan pl = plan_fwd_ws(a, workspace != nullptr ? workspace_bytes : 0);
  const uint16_t* vsrc = (const uint16_t*)a.v;
  if (pl.vt) {
    uint16_t* vt = (uint16_t*)((char*)workspace + pl.vt_off);
    const int64_t ntile = (a.nk + kBN - 1) / kBN;
    auto pack = a.head_dim == 64 ? (a.tiled ? vt_pack_kernel<64, true> : vt_pack_kernel<64, false>)
                                 : (a.tiled ? vt_pack_kernel<128, true> : vt_pack_kernel<128, false>);
    // heads split over gridDim.y until about 1,024 workgroups (1 when the tiles alone give that)
    const int hp = kPackThreads / a.head_dim;
    const int64_t hsplit = std::max<int64_t>(1, std::min<int64_t>((a.heads + hp - 1) / hp,
                                                                  (1024 + a.batch * ntile - 1) / (a.batch * ntile)));
    hipLaunchKernelGGL(pack, dim3((unsigned)(a.batch * ntile), (unsigned)hsplit), dim3(kPackThreads), 0, stream,
                       (const uint16_t*)a.v, vt, a.nk, a.heads, ntile, tg);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    vsrc = vt;
  }
  Work wk;
  Groups gp{1, 1, 0, 1};
  const int32_t *kcol = a.col_idx, *gmask = nullptr, *gcnt = nullptr;
  if (pl.grouped) {
    const int nbk = (int)((a.nk + a.block_k - 1) / a.block_k);
    const int64_t lists = (int64_t)a.n_slabs * pl.n_groups;
    char* ws = (char*)workspace;
    int32_t* gcol = (int32_t*)ws;
    int32_t* gmask_w = (int32_t*)(ws + align256(4 * (size_t)(lists * nbk)));
    int32_t* gcnt_w = (int32_t*)(ws + 2 * align256(4 * (size_t)(lists * nbk)));
    gmask = gmask_w;
    gcnt = gcnt_w;
    const hipError_t e = launch_group_union(a.row_ptr, a.col_idx, nbq, lists, pl.G, pl.n_groups, a.group_stride, nbk,
                                            gcol, gmask_w, gcnt_w, stream);
    if (e != hipSuccess) return e;
    gp = Groups{pl.G, pl.wpb, nbk, a.group_stride};
    kcol = gcol;
    wk.nbq = pl.n_groups;
    wk.mt_per_qb = 1;
  } else {
    const int bm = 32 * pl.nw / pl.ks;
    wk.nbq = nbq;
    wk.mt_per_qb = (a.block_q + bm - 1) / bm;
  }
  Split sp{nullptr, nullptr, a.batch * a.heads * a.nq, pl.splits};
  if (pl.splits > 1) {  // the partial outputs, after the union lists of a grouped plan
    char* base = (char*)workspace +
                 (pl.grouped ? union_bytes((int64_t)a.n_slabs * pl.n_groups, (a.nk + a.block_k - 1) / a.block_k) : 0);
    sp.o = (float*)base;
    sp.ml = (float*)(base + align256(4 * (size_t)(pl.splits * sp.rows * a.head_dim)));
  }
  wk.items = a.batch * a.heads * (int64_t)wk.nbq * wk.mt_per_qb * pl.splits;
  wk.per_xcd = (wk.items + 7) / 8;
  wk.chunk = xcd_run(a.nk, a.head_dim, 2);
  const dim3 grid((unsigned)(wk.per_xcd * 8));
  auto launch = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(pl.nw * kWave), 0, stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, vsrc, (uint16_t*)a.o, a.lse, a.nq, a.nk,
                       a.heads, a.block_q, a.block_k, a.row_ptr, kcol, gmask, gcnt, a.n_slabs, sl2, wk, gp, tg, sp);
  };
  // instantiation for (head_dim, plan, tiled, packed V^T)
  auto pick = [&](auto dc, auto tc, auto vc) {
    constexpr int D = decltype(dc)::value;
    constexpr bool TL = decltype(tc)::value;
    constexpr bool VT = decltype(vc)::value;
    if (pl.grouped) {
      if constexpr (!TL) {
        if (pl.tw == 2 && pl.nw == 12) return launch(attn_fwd_bf16_kernel<D, 1, 12, true, false, 2, false, VT>);
        if (pl.tw == 2) return launch(attn_fwd_bf16_kernel<D, 1, 8, true, false, 2, false, VT>);
      }
      if (pl.nw == 12) launch(attn_fwd_bf16_kernel<D, 1, 12, true, TL, 1, false, VT>);
      else if (pl.nw == 8) launch(attn_fwd_bf16_kernel<D, 1, 8, true, TL, 1, false, VT>);
      else launch(attn_fwd_bf16_kernel<D, 1, 4, true, TL, 1, false, VT>);
      return;
    }
    if (pl.splits > 1) {
      if (pl.ks == 2) launch(attn_fwd_bf16_kernel<D, 2, 4, false, TL, 1, true, VT>);
      else if (pl.nw == 12) launch(attn_fwd_bf16_kernel<D, 1, 12, false, TL, 1, true, VT>);
      else if (pl.nw == 8) launch(attn_fwd_bf16_kernel<D, 1, 8, false, TL, 1, true, VT>);
      else launch(attn_fwd_bf16_kernel<D, 1, 4, false, TL, 1, true, VT>);
      return;
    }
    if (pl.ks == 2) launch(attn_fwd_bf16_kernel<D, 2, 4, false, TL, 1, false, VT>);
    else if (pl.nw == 12) launch(attn_fwd_bf16_kernel<D, 1, 12, false, TL, 1, false, VT>);
    else if (pl.nw == 8) launch(attn_fwd_bf16_kernel<D, 1, 8, false, TL, 1, false, VT>);
    else launch(attn_fwd_bf16_kernel<D, 1, 4, false, TL, 1, false, VT>);
  };
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  if (a.head_dim == 64) {
    if (a.tiled) pl.vt ? pick(D64{}, Yes{}, Yes{}) : pick(D64{}, Yes{}, No{});
    else pl.vt ? pick(D64{}, No{}, Yes{}) : pick(D64{}, No{}, No{});
  } else {
    if (a.tiled) pl.vt ? pick(D128{}, Yes{}, Yes{}) : pick(D128{}, Yes{}, No{});
    else pl.vt ? pick(D128{}, No{}, Yes{}) : pick(D128{}, No{}, No{});
  }
  if (pl.splits > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t threads = sp.rows * (a.head_dim / 4);
    hipLaunchKernelGGL(a.head_dim == 64 ? split_merge_kernel<64> : split_merge_kernel<128>,
                       dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, sp.o, sp.ml, sp.n, sp.rows,
                       a.heads, a.nq, (uint16_t*)a.o, a.lse);
  }
  return hipGetLastError();
}

}  // namespace vsa

/*
 * vsa.h -- block-sparse softmax attention over a 3D (T x H x W) video-token grid,
 * for AMD Instinct MI355X (gfx950).  C ABI; plain pointers and sizes.
 *
 * The path: make 3D tiles contiguous (vsa_tile_reorder), build a block mask as a
 * CSR list of kept key blocks (vsa_mask_sta, vsa_mask_radial, vsa_mask_nabla; composed
 * with vsa_mask_sta_heads and vsa_mask_union),
 * then compute exact softmax(Q K^T * scale) V over the kept blocks only
 * (vsa_block_sparse_attn_fwd; vsa_tiled_attn_fwd folds the reorder into it;
 * vsa_radial_attn_fwd groups its work across frames) and its gradients
 * (vsa_block_sparse_attn_bwd).  vsa_block_mean_pool and vsa_block_sics are the
 * pooling and scoring passes on one tensor.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Token tensors are [batch, n_tokens, heads, head_dim], contiguous, head_dim
 *   fastest, in device memory.  Tokens are in raster order (t, h, w), w fastest,
 *   unless they went through vsa_tile_reorder.
 * - A block is a run of `block` consecutive tokens; the last block of a sequence
 *   may be ragged.  n_qblocks = ceil(nq / block_q), n_kblocks = ceil(nk / block_k).
 * - Token counts (nq, nk, n) of the calls on token tensors must be below 2^31 - 64
 *   (the kernels step through them in 31-bit arithmetic); larger ones give
 *   VSA_ERR_SHAPE.
 * - CSR mask: row r lists, in ascending order, the key blocks kept by query block
 *   r; row_ptr[n_rows + 1] holds absolute int32 offsets into col_idx, both in
 *   device memory.  A mask shared by all (batch, head) has n_rows = n_qblocks
 *   ("one slab"); a per-(batch, head) mask has n_rows = batch * heads * n_qblocks
 *   with row r = (b * heads + h) * n_qblocks + qblock.
 * - Ownership: the caller owns every buffer.  The library allocates no device
 *   memory, holds no mutable global state and is reentrant (except
 *   vsa_block_sparse_attn_fwd_static, whose workspace is a fixed device array).  Pointers are borrowed
 *   until the work enqueued on `stream` completes; every call is asynchronous and
 *   returns once its kernels are enqueued.
 * - Errors: every argument is validated on the host before anything is launched;
 *   on error nothing is launched and no output is touched.  A failure reported by
 *   the HIP runtime at launch maps to VSA_ERR_HIP.  Nothing is printed and no
 *   exception crosses the ABI.
 */
#ifndef VSA_H
#define VSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t vsa_status;
#define VSA_OK 0
#define VSA_ERR_NULL (-1)        /* a required pointer is NULL                              */
#define VSA_ERR_SHAPE (-2)       /* a size <= 0, inconsistent sizes, grid not divisible     */
#define VSA_ERR_DTYPE (-3)       /* dtype is not VSA_F32 or VSA_BF16                        */
#define VSA_ERR_PARAM (-4)       /* even / non-positive window, threshold outside (0, 1],   */
                                 /* topk < 0, forced range outside [0, n_kblocks], n_slabs  */
#define VSA_ERR_CAPACITY (-5)    /* col_capacity or workspace too small                     */
#define VSA_ERR_UNSUPPORTED (-6) /* head_dim not 64 / 128, misaligned pointer or row size   */
#define VSA_ERR_HIP (-7)         /* the HIP runtime reported an error at launch             */

enum { VSA_F32 = 0, VSA_BF16 = 1 };

/* Human-readable name of a status code (static string). */
const char* vsa_status_string(vsa_status s);

/*
 * vsa_tile_reorder -- permute whole token rows between raster order and
 * tile-major order.
 *
 * Sliding Tile Attention explainer (aibr.jp/archives/60739), sec. 2-3: the video
 * is processed in small rectangular 3D tiles, and organising the work per tile
 * (instead of per token) cuts memory traffic and redundancy.  Tile-major order
 * puts the tt*th*tw tokens of each tile next to each other, tiles in raster order
 * over the (T/tt, H/th, W/tw) tile grid, tokens raster inside a tile.  Position
 * p = ((it*NH + ih)*NW + iw)*V + (lt*th + lh)*tw + lw holds raster token
 * ((it*tt + lt)*H + ih*th + lh)*W + iw*tw + lw, with V = tt*th*tw.
 *
 * src, dst   device, [batch, T*H*W, row] rows of row_bytes bytes; must not overlap;
 *            16-byte aligned.
 * row_bytes  bytes per token row = heads * head_dim * element size; multiple of 16.
 * inverse    0: raster -> tile-major;  1: tile-major -> raster.
 * Errors: VSA_ERR_NULL, VSA_ERR_SHAPE (non-positive size, T/H/W not divisible by
 * tt/th/tw), VSA_ERR_UNSUPPORTED (row_bytes % 16, misalignment), VSA_ERR_HIP.
 */
vsa_status vsa_tile_reorder(const void* src, void* dst, int64_t batch,
                            int32_t T, int32_t H, int32_t W,
                            int32_t tt, int32_t th, int32_t tw,
                            int64_t row_bytes, int32_t inverse, hipStream_t stream);

/*
 * vsa_mask_sta -- sliding 3D tile window (one slab, shared by all batch/heads).
 *
 * Sliding Tile Attention explainer (aibr.jp/archives/60739), sec. 3: every query
 * tile attends the tiles of a window that slides with it (3D locality, sec. 1).
 * Query tile i keeps key tile j iff |i_t - j_t| <= wt/2, |i_h - j_h| <= wh/2 and
 * |i_w - j_w| <= ww/2 (tile coordinates; the window is centred and clipped at the
 * border).  Tiles are numbered in raster order over the tile grid, i.e. block j of
 * a tile-reordered sequence is tile j; block size = tt*th*tw.
 *
 * row_ptr   device, n_tiles + 1 ints;  col_idx  device, col_capacity ints.
 * col_capacity must be >= n_tiles * min(wt, NT) * min(wh, NH) * min(ww, NW).
 * Errors: VSA_ERR_NULL, VSA_ERR_SHAPE, VSA_ERR_PARAM (even or non-positive
 * window), VSA_ERR_CAPACITY, VSA_ERR_HIP.
 */
vsa_status vsa_mask_sta(int32_t T, int32_t H, int32_t W, int32_t tt, int32_t th, int32_t tw,
                        int32_t wt, int32_t wh, int32_t ww,
                        int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                        hipStream_t stream);

/*
 * vsa_mask_radial -- energy-decay radial mask over raster order (one slab).
 *
 * Radial Attention explainer (aibr.jp/archives/112136), sec. 2-3: dense between
 * nearby frames; the spatial window shrinks exponentially with temporal distance,
 * giving O(n log n) kept pairs.  Token pair (q, k), frames f = n / S, in-frame
 * index s = n % S, d = |f_q - f_k|, r = floor(log2 d): kept iff d <= 1 or
 * |s_q - s_k| * 2^r < S.  Block pair (I, J) is kept iff any of its token pairs
 * is.  N = T*S tokens, n_blocks = ceil(N / block) rows and columns.
 *
 * row_ptr   device, n_blocks + 1 ints;  col_idx  device, col_capacity ints.
 * col_capacity must be >= n_blocks * n_blocks (the exact count is only known on
 * the device).
 * Errors: VSA_ERR_NULL, VSA_ERR_SHAPE (non-positive sizes, N >= 2^31),
 * VSA_ERR_CAPACITY, VSA_ERR_HIP.
 */
vsa_status vsa_mask_radial(int32_t T, int32_t S, int32_t block,
                           int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                           hipStream_t stream);

/*
 * vsa_mask_sta_heads -- sliding 3D tile window with one window per head.
 *
 * Sliding Tile Attention explainer (aibr.jp/archives/60739), sec. 1: attention
 * heads specialise, so each head may use its own window; every slab is the
 * vsa_mask_sta mask of its head's window.  Slab s = b * heads + h (the per-head
 * slab order of vsa_block_sparse_attn_fwd), row r = s * n_tiles + tile.
 *
 * windows   host, heads * 3 ints (wt, wh, ww) per head, odd and positive.
 * heads     1 .. 256;  batch >= 1 (the heads' slabs repeat per batch entry).
 * row_ptr   device, batch * heads * n_tiles + 1 ints;  col_idx  device.
 * col_capacity must be >= batch * sum over heads of
 *   n_tiles * min(wt, NT) * min(wh, NH) * min(ww, NW).
 * Errors: VSA_ERR_NULL, VSA_ERR_SHAPE, VSA_ERR_PARAM (even or non-positive
 * window), VSA_ERR_UNSUPPORTED (more than 256 heads), VSA_ERR_CAPACITY,
 * VSA_ERR_HIP.
 */
vsa_status vsa_mask_sta_heads(int32_t T, int32_t H, int32_t W, int32_t tt, int32_t th, int32_t tw,
                              const int32_t* windows, int32_t heads, int64_t batch,
                              int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                              hipStream_t stream);

/*
 * vsa_mask_union -- row-by-row union of two block masks (e.g. NABLA with STA).
 *
 * NABLA explainer (aibr.jp/archives/124678), sec. 2 and 4: the NABLA mask works
 * alongside other accelerations and combines with them.  Output row r keeps key
 * block j iff row r of mask A or of mask B keeps it, in ascending order.  Masks
 * have n_qblocks rows per slab; a mask with one slab is shared by every slab of
 * the other, and the output has max(slabs_a, slabs_b) slabs.
 *
 * row_ptr_a/col_idx_a, row_ptr_b/col_idx_b  device CSR inputs; every row strictly
 *           ascending with values in [0, n_kblocks) (as the mask calls write
 *           them); the output is undefined otherwise.
 * row_ptr   device, max(slabs) * n_qblocks + 1 ints;  col_idx  device.
 * col_capacity must be >= max(slabs) * n_qblocks * n_kblocks.
 * Errors: VSA_ERR_NULL, VSA_ERR_SHAPE, VSA_ERR_PARAM (slab counts neither equal
 * nor 1), VSA_ERR_CAPACITY, VSA_ERR_HIP.
 */
vsa_status vsa_mask_union(int64_t n_qblocks, int32_t n_kblocks,
                          const int32_t* row_ptr_a, const int32_t* col_idx_a, int64_t slabs_a,
                          const int32_t* row_ptr_b, const int32_t* col_idx_b, int64_t slabs_b,
                          int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                          hipStream_t stream);

/*
 * vsa_block_sics -- SICS block scores: sum of intra-block cosine similarities.
 *
 * SPADE summary (gist.science/ja/paper/2608.03335), "The solution" part 2: the
 * scheme step groups tokens into blocks and scores how strongly each group's
 * members agree.  Score of block i of head h = sum over all ordered token pairs
 * (a, b) of the block, a = b included, of cos(x_a, x_b) = |sum_a x_a / |x_a||^2;
 * a zero token row contributes nothing.  Computed in fp64.  Which tensor to score
 * (Q or K) and how to select blocks from the scores are the caller's choice; the
 * page states neither.
 *
 * x        device, [batch, n, heads, head_dim] (dtype VSA_F32 or VSA_BF16), 16-byte
 *          aligned; head_dim 64 or 128.
 * scores   device, [batch, heads, ceil(n / block)] doubles.
 * Errors: VSA_ERR_NULL, VSA_ERR_DTYPE, VSA_ERR_SHAPE, VSA_ERR_UNSUPPORTED
 * (head_dim, alignment), VSA_ERR_HIP.
 */
vsa_status vsa_block_sics(const void* x, int32_t dtype, int64_t batch, int32_t heads, int32_t head_dim,
                          int64_t n, int32_t block, double* scores, hipStream_t stream);

/*
 * KV-cache compaction for chunked autoregressive generation.
 *
 * Sparse Forcing summary (gist.science/ja/paper/2604.21221), parts 2-3: anchor
 * blocks are kept as persistent memory and recent blocks only where needed; the
 * rest of the past is not stored (42% less memory on the page).  A (batch, head)
 * keeps the union of the key blocks its mask rows keep; the compact cache keeps
 * the [batch, tokens, heads, head_dim] layout, each head's kept full blocks packed
 * from slot 0 in ascending order and a kept ragged last block in one shared tail
 * slot after the largest head's full blocks.  With the mask rewritten onto the
 * slots, attention over the compact cache equals attention over the full cache.
 *
 * vsa_kv_plan -- slot map of each mask slab.
 *   row_ptr/col_idx  device CSR mask, n_slabs * n_qblocks rows (1 slab = shared).
 *   slot   device, n_slabs * ceil(nk / block_k) ints out: slot of each key block,
 *          -1 if no row of the slab keeps it.
 *   info   device, 2 + 2 * n_slabs ints out: info[0] = full blocks of the largest
 *          slab (= the tail slot), info[1] = 1 if a slab keeps a ragged last block;
 *          the rest is per-slab scratch.  The compact cache holds
 *          info[0] * block_k + (info[1] ? nk % block_k : 0) tokens.
 *   Errors: VSA_ERR_NULL, VSA_ERR_SHAPE, VSA_ERR_HIP.
 *
 * vsa_kv_gather -- copy the kept blocks of x [batch, nk, heads, head_dim] into out
 *   [batch, n_out, heads, head_dim] (same dtype, 16-byte aligned); slot/n_slabs as
 *   planned (n_slabs 1 or batch * heads).  Slots no kept block maps to are not
 *   written; writes past n_out are dropped, so pass n_out from info.
 *   Errors: VSA_ERR_NULL, VSA_ERR_DTYPE, VSA_ERR_SHAPE, VSA_ERR_PARAM (n_slabs),
 *   VSA_ERR_UNSUPPORTED (head_dim, alignment), VSA_ERR_HIP.
 *
 * vsa_mask_remap -- col_out[e] = slot of col_idx[e] in its row's slab; row_ptr is
 *   unchanged and rows stay ascending.  col_out device, row_ptr[n_rows] ints.
 *   Errors: VSA_ERR_NULL, VSA_ERR_SHAPE, VSA_ERR_HIP.
 */
vsa_status vsa_kv_plan(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_slabs, int64_t n_qblocks,
                       int64_t nk, int32_t block_k, int32_t* slot, int32_t* info, hipStream_t stream);
vsa_status vsa_kv_gather(const void* x, int32_t dtype, int64_t batch, int32_t heads, int32_t head_dim,
                         int64_t nk, int32_t block_k, const int32_t* slot, int64_t n_slabs, void* out,
                         int64_t n_out, hipStream_t stream);
vsa_status vsa_mask_remap(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_slabs, int64_t n_qblocks,
                          const int32_t* slot, int32_t n_kblocks, int32_t* col_out, hipStream_t stream);

/*
 * vsa_block_mean_pool -- mean of each block's token rows, per head, in fp64.
 *
 * NABLA explainer (aibr.jp/archives/124678), sec. 3: Q and K are average-pooled per
 * block before the small attention map is formed.  This is that pooling step on one
 * tensor (vsa_mask_nabla runs the same kernel on Q and K): out[b, i, h, :] = the mean
 * over the valid tokens t of block i (the last block may be ragged) of x[b, t, h, :]
 * (block-major, the order of the token tensor itself).
 * The sums are accumulated in fp64 (exact for bf16 rows) and divided once by the
 * block's token count.
 *
 * x     device, [batch, n, heads, head_dim], dtype VSA_BF16 or VSA_F32, 16-byte aligned.
 * out   device, [batch, ceil(n / block), heads, head_dim] doubles, 8-byte aligned.
 * Errors: VSA_ERR_NULL, VSA_ERR_DTYPE, VSA_ERR_SHAPE (non-positive sizes, batch above
 * 65535, ceil(n / block) * ceil(heads * head_dim / 512) above 2^31 - 1),
 * VSA_ERR_UNSUPPORTED (head_dim not 64/128, alignment), VSA_ERR_HIP.
 */
vsa_status vsa_block_mean_pool(const void* x, int32_t dtype, int64_t batch, int32_t heads, int32_t head_dim,
                               int64_t n, int32_t block, double* out, hipStream_t stream);

/* Selection rule of vsa_mask_nabla. */
typedef struct {
  double cdf_threshold;   /* NABLA cut, in (0, 1]; used when topk == 0           */
  int32_t topk;           /* > 0: keep the top-k non-forced blocks by pooled logit */
  int32_t n_forced;       /* number of [lo, hi) key-block ranges always kept      */
  const int32_t* forced;  /* host array of 2 * n_forced ints (lo0, hi0, lo1, ...)  */
} vsa_select;

/*
 * vsa_mask_nabla -- dynamic block mask from mean-pooled Q and K, one slab per
 * (batch, head).
 *
 * NABLA explainer (aibr.jp/archives/124678), sec. 3: Q and K are average-pooled
 * per block, a small full attention map is computed from the pooled vectors, and
 * each row is binarised by a threshold on its cumulative distribution; the mask
 * adapts per sample (sec. 1).  With pooled means Qp (over the valid tokens of
 * each query block) and Kp, Z = Qp Kp^T * scale and p = softmax(Z) per row (fp64
 * throughout); the row is sorted by p descending (ties: lower block first) and
 * the shortest prefix whose running sum reaches cdf_threshold is kept (the
 * crossing block included; threshold 1 keeps every block).
 * With topk > 0 (Sparse Forcing summary, gist.science/ja/paper/2604.21221, part
 * 2: persistent anchors, recent frames, and only the needed past blocks) the
 * forced ranges are always kept and, of the other blocks, the topk with the
 * largest Z (ties: lower block first).
 *
 * q [batch, nq, heads, head_dim], k [batch, nk, heads, head_dim], device, dtype.
 * row_ptr   device, batch*heads*n_qblocks + 1 ints;  col_idx device.
 * col_capacity must be >= batch*heads*n_qblocks*n_kblocks.
 * workspace device scratch; when workspace == NULL the call only writes the
 *           required size to *workspace_bytes and returns VSA_OK.
 * Errors: VSA_ERR_NULL, VSA_ERR_SHAPE (also batch above 65535), VSA_ERR_DTYPE, VSA_ERR_PARAM,
 * VSA_ERR_CAPACITY (col_capacity or *workspace_bytes too small),
 * VSA_ERR_UNSUPPORTED (head_dim, alignment, n_kblocks > 4096), VSA_ERR_HIP.
 */
vsa_status vsa_mask_nabla(const void* q, const void* k, int32_t dtype,
                          int64_t batch, int32_t heads, int32_t head_dim,
                          int64_t nq, int64_t nk, int32_t block_q, int32_t block_k,
                          double scale, const vsa_select* sel,
                          int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                          void* workspace, size_t* workspace_bytes, hipStream_t stream);

/*
 * vsa_block_sparse_attn_fwd -- exact softmax attention over the kept blocks.
 *
 * Every page replaces full 3D attention (all tokens against all tokens, quadratic
 * cost; Radial Attention explainer sec. 1, Sliding Tile Attention explainer sec.
 * 1, NABLA explainer sec. 1) by attention over a subset of blocks, computed
 * head-wise (SPADE summary, gist.science/ja/paper/2608.03335, "The solution" part
 * 3).  For a query token of block i with kept key blocks J_i:
 *   o = sum_j softmax_j(q . k_j * scale) v_j over every valid token of J_i,
 *   lse = ln sum_j exp(q . k_j * scale).
 * A row with no kept block gives o = 0 and lse = -inf.  bf16 inputs are
 * multiplied on the matrix cores with fp32 accumulation and the probabilities are
 * rounded to bf16 before P V; fp32 inputs stay fp32 throughout.
 *
 * q, o [batch, nq, heads, head_dim]; k, v [batch, nk, heads, head_dim]; device,
 * dtype, 16-byte aligned.  lse: NULL or device [batch, heads, nq] fp32.
 * row_ptr/col_idx: CSR with n_slabs = 1 (shared) or batch*heads slabs.
 * scale: finite and > 0 (the usual 1/sqrt(head_dim)).
 * workspace / workspace_bytes: call with workspace = NULL and workspace_bytes set
 * to get the size.  bf16 query blocks of at most 128 rows are then run grouped:
 * several consecutive query blocks share a workgroup and walk the union of their
 * kept key blocks, so one copy of a key tile serves more query rows.  When the rows
 * are too few to fill the chip once (fewer workgroups than the chip runs at a time:
 * e.g. a few heads of short query blocks over a long key sequence), each row's
 * kept-block list is instead cut into up to 8 contiguous chunks walked by separate workgroups, whose
 * fp32 partial outputs (with their running maximum and row sum) a second kernel
 * adds in chunk order: the result is deterministic and equals the unsplit run to
 * rounding.  Third, when key blocks are a multiple of 64 tokens and nq >= nk (every
 * key tile is then read by many query blocks), V is first copied transposed into the
 * workspace, [batch, heads, ceil(nk / 64), head_dim, 64], so the P V product reads it
 * 16 bytes per lane.  The workspace (device, 256-byte aligned) holds, in this order,
 * the union lists or the partial outputs, then the transposed V; the size query
 * reports all of it.  A smaller workspace is used as far as it goes: the transposed V
 * only if it fits after the lists or partials, and with workspace = NULL, or smaller
 * than the lists or partials, the call runs neither grouped nor split.  Runs with the
 * same V layout and tile walk give the same result bit for bit (grouped and ungrouped
 * query blocks of 65 to 128 rows); the transposed V and the two-wave split of each key
 * tile for ungrouped blocks of at most 64 rows change the summation order, so across
 * those the results agree to rounding only.
 * bf16 token rows must be below 2^24 bytes (heads * head_dim * 2 < 2^24, i.e. at most
 * 65,535 heads at head_dim 128); the kernels address a tile's rows in 24-bit arithmetic.
 * Errors: VSA_ERR_NULL, VSA_ERR_SHAPE, VSA_ERR_DTYPE, VSA_ERR_PARAM (n_slabs, scale),
 * VSA_ERR_UNSUPPORTED (head_dim not 64/128, misalignment, bf16 row size), VSA_ERR_CAPACITY,
 * VSA_ERR_HIP.  The CSR contents are trusted: column indices must lie in
 * [0, n_kblocks) and row_ptr must be non-decreasing.
 */
vsa_status vsa_block_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int32_t dtype, int64_t batch, int32_t heads,
                                     int32_t head_dim, int64_t nq, int64_t nk,
                                     int32_t block_q, int32_t block_k,
                                     const int32_t* row_ptr, const int32_t* col_idx,
                                     int32_t n_slabs, float scale,
                                     void* workspace, size_t* workspace_bytes,
                                     hipStream_t stream);

/*
 * vsa_block_sparse_attn_fwd_static -- vsa_block_sparse_attn_fwd with no workspace
 * argument and no allocation, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The workspace the forward would ask for (union lists of grouped query blocks, or
 * the partial outputs of split key streams, then the transposed V when it fits in
 * what is left) is taken from a 64 MiB array that the library holds on every GPU it
 * runs on until the process ends; every other argument and the result are those of
 * vsa_block_sparse_attn_fwd with a workspace of that size.  The array
 * is state shared by every call on a GPU: calls that overlap on one GPU (two streams,
 * or two threads) race and must be serialised by the caller.  Nothing in it needs to
 * start at zero (every value is written before it is read), and it keeps the last
 * call's contents.  The call allocates nothing: no hipMalloc, hipFree or allocating
 * library routine.
 * Errors: as for vsa_block_sparse_attn_fwd; VSA_ERR_CAPACITY (checked before anything
 * touches the device) when the union lists or partial outputs alone need more than
 * 64 MiB (the transposed V is optional and skipped when it does not fit).
 */
vsa_status vsa_block_sparse_attn_fwd_static(const void* q, const void* k, const void* v, void* o,
                                            float* lse, int32_t dtype, int64_t batch, int32_t heads,
                                            int32_t head_dim, int64_t nq, int64_t nk, int32_t block_q,
                                            int32_t block_k, const int32_t* row_ptr,
                                            const int32_t* col_idx, int32_t n_slabs, float scale,
                                            hipStream_t stream);

/*
 * vsa_radial_attn_fwd -- the forward above, for masks over raster-order frames, with
 * query blocks grouped across frames.
 *
 * Radial Attention explainer (aibr.jp/archives/112136), sec. 2-3: the spatial window
 * shrinks with temporal distance, so far from its own frame a query block keeps only
 * the key blocks around its own place in each other frame -- nearly the same key blocks
 * as the query blocks at that place in the neighbouring frames.  With a workspace and
 * bf16 query blocks of at most 128 rows, this call groups query blocks P apart (P =
 * frame_tokens / block_q, rounded down, at least 1: the same place in consecutive
 * frames) instead of consecutive ones, so the union of kept key blocks that a group
 * walks is close to one row's.  Any CSR mask is accepted and the result is the same as
 * vsa_block_sparse_attn_fwd's (bit for bit where both group blocks of 65 to 128 rows);
 * only the work order differs.  The workspace size must be queried from this call.
 *
 * frame_tokens  tokens per frame (> 0); every other argument as for
 *               vsa_block_sparse_attn_fwd.
 * Errors: as for vsa_block_sparse_attn_fwd; VSA_ERR_SHAPE also for frame_tokens <= 0.
 */
vsa_status vsa_radial_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                               int32_t dtype, int64_t batch, int32_t heads, int32_t head_dim,
                               int64_t nq, int64_t nk, int32_t block_q, int32_t block_k,
                               int64_t frame_tokens, const int32_t* row_ptr, const int32_t* col_idx,
                               int32_t n_slabs, float scale, void* workspace, size_t* workspace_bytes,
                               hipStream_t stream);

/*
 * vsa_tiled_attn_fwd -- the forward above on raster-order tokens of a 3D grid,
 * with the tiles as blocks and no reorder pass.
 *
 * Sliding Tile Attention explainer (aibr.jp/archives/60739), sec. 1-3: sliding
 * tile attention replaces full 3D attention as a drop-in, Q, K and V in, O out,
 * same shape; the tile-major order (vsa_tile_reorder) is what makes each tile's
 * tokens one block.  This call reads q, k, v and writes o and lse in raster order
 * and applies the tile-major permutation to the row addresses inside the kernel:
 * the result equals vsa_tile_reorder of q, k, v, then vsa_block_sparse_attn_fwd
 * with block_q = block_k = tt*th*tw, then the inverse reorder of o (and of lse),
 * bit for bit, without moving the token tensors through HBM twice.
 *
 * q, k, v, o  device, [batch, T*H*W, heads, head_dim] in raster order, dtype,
 *             16-byte aligned.  lse: NULL or device [batch, heads, T*H*W] fp32, raster
 *             order.
 * row_ptr/col_idx  CSR over the tile-major tiles (n_tiles = T/tt * H/th * W/tw rows
 *             per slab; vsa_mask_sta's output), n_slabs = 1 or batch*heads.
 * workspace / workspace_bytes, scale: as for vsa_block_sparse_attn_fwd (grouping, the
 * split of small problems and the transposed V included; here the transposed copy is
 * in tile-major key order).  The bit-for-bit equality above holds between calls given
 * the workspace each one asks for, or none.
 * The tile's h-w plane must nest with the kernel's 64-token copy tile: th*tw a
 * multiple of 64 with tw dividing 64 or a multiple of 64, or th*tw dividing 64 (the
 * 6x8x8 and 1x8x8 tiles of the pages' video models qualify), and a tile holds at
 * most 4096 tokens.  For bf16 the 64 tokens of one copy tile must also lie within
 * 2^24 rows and 4 GiB of the copy tile's first token: span < 2^24 and
 * (span + 1) * heads * head_dim * 2 < 2^32, with span = (64/tw - 1) W + tw - 1, 63,
 * or (64/(th tw) - 1) H W + (th - 1) W + tw - 1 for the three plane shapes above.
 * Errors: VSA_ERR_NULL, VSA_ERR_SHAPE (non-positive sizes, T/H/W not divisible by
 * tt/th/tw, T*H*W >= 2^31 - 64), VSA_ERR_DTYPE, VSA_ERR_PARAM (n_slabs, scale),
 * VSA_ERR_UNSUPPORTED (head_dim not 64/128, misalignment, tile shape or size, copy-tile
 * span), VSA_ERR_HIP.
 */
vsa_status vsa_tiled_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                              int32_t dtype, int64_t batch, int32_t heads, int32_t head_dim,
                              int32_t T, int32_t H, int32_t W, int32_t tt, int32_t th, int32_t tw,
                              const int32_t* row_ptr, const int32_t* col_idx, int32_t n_slabs,
                              float scale, void* workspace, size_t* workspace_bytes,
                              hipStream_t stream);

/*
 * vsa_block_sparse_attn_bwd -- gradients of the forward above.
 *
 * Radial Attention explainer (aibr.jp/archives/112136), sec. 4: the sparse
 * pattern saves training as well as inference time, so the path has a backward
 * pass.  For L = sum(dout * o) with o = vsa_block_sparse_attn_fwd(q, k, v) over
 * the same mask, with p = exp(q . k * scale - lse) and D_i = sum_d dout_i o_i:
 *   dv_j = sum_i p_ij dout_i,  dp_ij = dout_i . v_j,  ds_ij = p_ij (dp_ij - D_i),
 *   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
 * sums over the kept (query, key) pairs only.  bf16 inputs run on the matrix
 * cores with p and ds rounded to bf16; fp32 inputs stay fp32.  The result is
 * deterministic (no atomics): key gradients walk a transposed copy of the mask.
 *
 * q, o, dout [batch, nq, heads, head_dim]; k, v [batch, nk, heads, head_dim];
 *          device, dtype, 16-byte aligned; o and lse as written by the forward.
 * dq, dk, dv  device fp32 outputs with the shapes of q, k, v, 16-byte aligned;
 *          rows no kept pair touches get 0.
 * row_ptr/col_idx, n_slabs, scale: as for the forward.
 * workspace: device, 256-byte aligned; call with workspace = NULL to get the
 *          size in *workspace_bytes (fp32 D per query, the transposed mask sized
 *          for n_slabs * n_qblocks * n_kblocks entries, and for bf16 key blocks of
 *          <= 64 keys the union lists of the grouped dK/dV pass).
 * bf16 token rows must be below 2^24 bytes, as for the forward.
 * Errors: VSA_ERR_NULL, VSA_ERR_SHAPE, VSA_ERR_DTYPE, VSA_ERR_PARAM (n_slabs,
 * scale), VSA_ERR_UNSUPPORTED (head_dim, alignment, bf16 row size), VSA_ERR_CAPACITY
 * (workspace_bytes smaller than the query), VSA_ERR_HIP.
 */
vsa_status vsa_block_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                     const void* dout, const float* lse, float* dq, float* dk, float* dv,
                                     int32_t dtype, int64_t batch, int32_t heads, int32_t head_dim,
                                     int64_t nq, int64_t nk, int32_t block_q, int32_t block_k,
                                     const int32_t* row_ptr, const int32_t* col_idx, int32_t n_slabs,
                                     float scale, void* workspace, size_t* workspace_bytes,
                                     hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* VSA_H */

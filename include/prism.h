/*
 * prism.h -- C ABI of a MI355X (gfx950) library for Prism dynamic sparse
 * video self-attention: one attention layer over the video tokens of a
 * T x H x W latent grid, for the heads held by one GPU.
 *
 * Source: the Prism pages ("Prism: Dynamic Sparse Attention for Native 2K
 * Joint Video-Audio Generation Model Training").  Citations below name the
 * page and the section on it:
 *   [pt/IC]  Portuguese reading guide (xyznot.com/pt), "Ideias centrais"
 *   [pt/M1]  same page, "Método", part 1 (variation indicator)
 *   [pt/M2]  same page, "Método", part 2 (block volume and shape)
 *   [pt/M3]  same page, "Método", part 3 (hybrid Top-k / Top-p attention)
 *   [zh/FAQ] Chinese reading guide (xyznot.com/zh), "常见问题"
 *   [blog/4] sd114.wiki post, "工作原理", step 4
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers unless stated otherwise; the
 *   caller owns every buffer.  The library never allocates device memory;
 *   scratch comes from a caller-supplied workspace.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *   Only prism_select_blocks synchronises the stream (it reads the number of
 *   blocks and of selected index entries back to the host).
 * - Token order "THW": token n = (t * H + h) * W + w.  A THW tensor element
 *   (head, n, c) lives at  head * head_stride + n * token_stride + c.
 * - Block order: the permutation of prism_plan_shapes.  Block-order arrays
 *   are dense: element (head, p, c) at (head * N + p) * head_dim + c.
 * - bf16 values are uint16_t bit patterns of bfloat16.
 * - Every call validates its arguments (pointers, sizes, strides,
 *   hyper-parameters) before it launches anything, and returns PRISM_OK or a
 *   negative status; nothing is written on a validation error.  The
 *   contents of a block index (perm, blk_start, n_blocks and the block
 *   lists) are trusted by prism_attn_fwd and prism_attn_bwd, which read them
 *   on the device: an index written by prism_plan_shapes and
 *   prism_select_blocks is valid by construction; one from elsewhere is
 *   checked on a host copy with prism_check_index first (a malformed index
 *   makes the attention kernels read and write out of bounds).  NaN or Inf
 *   inputs give undefined results.
 * - The library keeps no state between calls; calls on different streams
 *   with disjoint outputs are independent.
 */
#ifndef PRISM_H
#define PRISM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t prism_bf16;
typedef void *prism_stream;

enum prism_status {
  PRISM_OK = 0,
  PRISM_EINVAL = -1,     /* NULL pointer, non-positive size, bad stride, grid too large */
  PRISM_EGRID = -2,      /* T, H or W not a positive multiple of 8 (zones do not overlap [pt/IC]) */
  PRISM_EDIM = -3,       /* head_dim not 64 or 128 */
  PRISM_EPARAM = -4,     /* eps <= 0, tau256 > tau128, top_k < 1, top_p or density_cap outside (0, 1], scale < 0, bad variant or pass_heads < 0 */
  PRISM_ECAPACITY = -5,  /* col_cap smaller than the number of selected (query block, key block) pairs */
  PRISM_EWORKSPACE = -6, /* workspace NULL-with-size or too small */
  PRISM_EHIP = -7,       /* a HIP runtime call failed */
  PRISM_EINDEX = -8      /* prism_check_index: the block index breaks an invariant */
};

/* The latent grid and the head layout of the THW tensors. */
typedef struct prism_problem {
  int32_t T, H, W;      /* grid; each a positive multiple of 8; N = T*H*W <= 1,048,576 (PRISM_EINVAL above) */
  int32_t heads;        /* heads handled by this call, >= 1 */
  int32_t head_dim;     /* D: 64 or 128 */
  int64_t head_stride;  /* elements between heads in THW tensors (>= 0) */
  int64_t token_stride; /* elements between tokens in THW tensors (>= head_dim) */
} prism_problem;

/* Variant switches (prism_params.variant, bitwise OR; 0 = the method as on the pages). */
enum prism_variant {
  PRISM_VARIANT_FIXED_SHAPE = 1,   /* every zone uses shape index `fixed_shape` (fixed-block baseline) */
  PRISM_VARIANT_TOPK_ONLY = 2,     /* S_i = Top-k only */
  PRISM_VARIANT_TOPP_ONLY = 4,     /* S_i = Top-p only (at least one block) */
  PRISM_VARIANT_VISUAL_ONLY = 8,   /* drop the audio term: g_d = r_v,d + eps */
  PRISM_VARIANT_AUDIO_ONLY = 16,   /* drop the video ratio: g_d = a-bar v-hat_a,d + eps */
  PRISM_VARIANT_RHO_MAX_AUDIO = 32 /* density max(rho, a-bar) instead of rho */
};

/* Hyper-parameters ([pt/M1], [pt/M2], [pt/M3]). */
typedef struct prism_params {
  double eps;          /* epsilon added to g_d, > 0 (pages: "+eps"; default 1e-6) */
  double tau128;       /* density below which a zone uses volume 128 (0.5 [pt/M2]) */
  double tau256;       /* density below which a zone uses volume 256 (0.25 [pt/M2]); tau256 <= tau128 */
  int32_t top_k;       /* k of Top-k, >= 1 */
  int32_t variant;     /* prism_variant bits */
  double top_p;        /* p of Top-p, in (0, 1]; 1 selects every block */
  double density_cap;  /* in (0, 1]; at most floor(cap * N) key tokens per query block beyond Top-k; 1 = none */
  double scale;        /* softmax scale of block scores and attention; 0 -> 1/sqrt(head_dim) */
  int32_t fixed_shape; /* shape index 0..15 for PRISM_VARIANT_FIXED_SHAPE */
  int32_t pass_heads;  /* prism_infer_fwd: heads per pass, >= 0; 0 = automatic */
} prism_params;

/* Candidate shapes, index 0..15: edges in {2,4,8}, volume in {64,128,256}
 * ([pt/IC]: 16 candidates), ordered by volume, then (b_T, b_H, b_W):
 *  64: 0 2x4x8, 1 2x8x4, 2 4x2x8, 3 4x4x4, 4 4x8x2, 5 8x2x4, 6 8x4x2
 * 128: 7 2x8x8, 8 4x4x8, 9 4x8x4, 10 8x2x8, 11 8x4x4, 12 8x8x2
 * 256: 13 4x8x8, 14 8x4x8, 15 8x8x4 */

/*
 * prism_zone_stats -- variation indicator of every 8x8x8 macro-zone
 * ([pt/IC] zones; [pt/M1] sigma^2_v,d, r_v,d, a-bar, v-hat_a,d, g_d;
 * [pt/M2] density rho).
 *
 * v      THW bf16 [heads] x [N] x [D]: the layer's value features.
 * a      float [N], shared by all heads: the cached audio-to-video
 *        cross-attention output norms of the previous layer
 *        (a_{t,h,w} = |h-hat_{t,h,w}|_2); NULL means no audio (all zero).
 * zstats double [heads][Z][8] (out): sigma^2_v,T, sigma^2_v,H, sigma^2_v,W
 *        (variance over the 8 slice means along each axis, channel
 *        averaged), sigma^2_a,T/H/W (same for a), mu_a (zone mean of a),
 *        a-bar (min-max normalised mu_a over the zones).
 * g      double [heads][Z][3] (out): g_d = r_v,d + a-bar v-hat_a,d + eps.
 * rho    double [heads][Z] (out): sum_d sigma^2_v,d over its maximum in the head.
 * Zone m = (t/8 * H/8 + h/8) * W/8 + w/8, Z = N / 512.  Statistics in float64.
 */
int prism_zone_stats(const prism_problem *prob, const prism_params *par, const prism_bf16 *v, const float *a,
                     double *zstats, double *g, double *rho, prism_stream stream);

/*
 * prism_plan_shapes -- block volume, block shape and token permutation
 * ([pt/M2]: B(m) from rho against tau_128 / tau_256; l*_d; nearest
 * candidate of that volume in log2 distance, lowest index on exact ties).
 *
 * g, rho     from prism_zone_stats.
 * shape_id   uint8 [heads][Z] (out): chosen candidate index.
 * perm       int32 [heads][N] (out): block-order position p -> THW token.
 *            Zones ascending; inside a zone its blocks in raster order (T
 *            outermost); inside a block its tokens in raster order.
 * blk_start  int32 [heads][N/64 + 1] (out): start of each block in units
 *            of 64 tokens (every block size is a multiple of 64 [zh/FAQ]);
 *            entries past n_blocks hold N/64.
 * n_blocks   int32 [heads] (out, device): blocks per head, N/256..N/64.
 */
int prism_plan_shapes(const prism_problem *prob, const prism_params *par, const double *g, const double *rho,
                      uint8_t *shape_id, int32_t *perm, int32_t *blk_start, int32_t *n_blocks, prism_stream stream);

/*
 * prism_select_blocks -- permute Q/K/V into block order, mean-pool query
 * and key blocks, score them and build the attended set
 * S_i = Top-k(P_i, k) U Top-p(P_i, p) of every query block ([pt/M3]).
 *
 * q, k, v     THW bf16 inputs.
 * perm, blk_start, n_blocks   from prism_plan_shapes.
 * qp, kp, vp  bf16 operand buffers (out), each heads * N * D values: the
 *             rows in block order, grouped in tiles of 64 rows; inside a tile
 *             row r is contiguous (D values) but its 16-byte chunk c (values
 *             8c .. 8c+7) is stored at chunk position c ^ f(r), with
 *             f(r) = ((r&3)<<2) | (((r>>2)&1)<<1) | ((r>>3)&1) for D = 128 and
 *             f(r) = (((r>>1)&1)<<2) | (((r>>2)&1)<<1) | ((r>>3)&1) for D = 64.
 *             Element (head, p, c) is therefore at
 *             (head * N + p) * D + 8 * ((c / 8) ^ f(p % 64)) + c % 8.
 * row_ptr     int32 [heads][N/64 + 1] (out): CSR row pointers of the
 *             query-major block index, offsets into col_idx counted over
 *             all heads (head h starts at the sum of the earlier heads'
 *             counts); entries past n_blocks repeat the head's end.
 * col_idx     int32 [col_cap] (out): selected key blocks of each row,
 *             ascending, block indices local to the head.
 * col_cap     capacity of col_idx and of t_col_idx, in entries.
 * t_row_ptr, t_col_idx   (out) the key-major transpose, same layout: for
 *             each key block, the query blocks that selected it, ascending.
 * nnz_host    HOST int64 [heads] (out): selected pairs per head.
 * ws, ws_bytes  workspace; with ws == NULL the call only stores the size it
 *             needs in *ws_bytes and returns PRISM_OK.
 * Returns PRISM_ECAPACITY when sum(nnz) > col_cap: nnz_host then holds the
 * counts, the permuted operands are written and the index is not.
 * Block scores s_ij = scale * Qbar_i . Kbar_j and P_i are float64; the
 * block order is (s descending, index ascending); the density cap trims only
 * the Top-p extension.  Synchronises the stream.
 */
int prism_select_blocks(const prism_problem *prob, const prism_params *par, const prism_bf16 *q,
                        const prism_bf16 *k, const prism_bf16 *v, const int32_t *perm, const int32_t *blk_start,
                        const int32_t *n_blocks, prism_bf16 *qp, prism_bf16 *kp, prism_bf16 *vp, int32_t *row_ptr,
                        int32_t *col_idx, int64_t col_cap, int32_t *t_row_ptr, int32_t *t_col_idx,
                        int64_t *nnz_host, void *ws, size_t *ws_bytes, prism_stream stream);

/*
 * prism_attn_fwd -- online-softmax attention of every query token over the
 * key tokens of its block's S_i only ([pt/M3]), scattered back to THW
 * order ([blog/4]).  No causal mask.
 *
 * qp, kp, vp  operand buffers from prism_select_blocks.
 * o           THW bf16 (out).
 * o_lo        bf16 [heads][N][D] (out, optional: NULL = not written), block
 *             order, contiguous: the low part of each output value,
 *             bf16(O - o) with O the float32 result, so that o + o_lo holds O
 *             to about 16 significant bits.  prism_attn_bwd takes it to form
 *             rowsum(dO * O) without the bf16 rounding of o (that rounding,
 *             up to 2^-8 relative, otherwise reaches every dS and moves dQ by about
 *             0.6-0.9% relative L2 on the test workloads).
 * lse         float [heads][N] (out), block order: natural-log log-sum-exp
 *             of each query row's scaled scores (kept for the backward).
 * ws, ws_bytes  workspace (the work-queue counters of the persistent
 *             kernel and its longest-first queue order, 256 B + about 6 B per
 *             64-token tile; size query as in prism_select_blocks).
 * bf16 MFMA products, float32 softmax and accumulation.  Calls that share a
 * workspace must not run concurrently.
 */
int prism_attn_fwd(const prism_problem *prob, const prism_params *par, const prism_bf16 *qp, const prism_bf16 *kp,
                   const prism_bf16 *vp, const int32_t *perm, const int32_t *blk_start, const int32_t *n_blocks,
                   const int32_t *row_ptr, const int32_t *col_idx, prism_bf16 *o, prism_bf16 *o_lo, float *lse,
                   void *ws, size_t *ws_bytes, prism_stream stream);

/*
 * prism_attn_fwd_noalloc -- prism_attn_fwd without a workspace argument, for
 * callers that cannot allocate device memory around the call (work under
 * stream capture, tight serving loops, harnesses that forbid allocation).
 * Its scratch (the work-queue counters and the longest-first queue order:
 * 256 B plus 6 B per 64-token tile of all heads) is a static 4 MiB device
 * array of the library, one copy per GPU, held until the process ends.  A
 * problem needing more (heads * N / 64 above about 699,000) returns
 * PRISM_EWORKSPACE before anything runs.  Every call on one GPU shares that
 * GPU's array and the array keeps the last call's contents (the counters are
 * cleared by a kernel at every call): calls that overlap in time on one GPU
 * (other streams, other host threads) race, so the caller serialises them.
 * Other arguments, results and errors as prism_attn_fwd; no allocating
 * routine is called.
 */
int prism_attn_fwd_noalloc(const prism_problem *prob, const prism_params *par, const prism_bf16 *qp,
                           const prism_bf16 *kp, const prism_bf16 *vp, const int32_t *perm, const int32_t *blk_start,
                           const int32_t *n_blocks, const int32_t *row_ptr, const int32_t *col_idx, prism_bf16 *o,
                           prism_bf16 *o_lo, float *lse, prism_stream stream);

/*
 * prism_attn_bwd -- gradients of the sparse attention with respect to Q, K
 * and V, through the selected blocks only; the zone statistics, shapes and
 * P_i are constants ([zh/FAQ]).
 *
 * o, dout     THW bf16: forward output and upstream gradient.
 * o_lo        the low parts of o from prism_attn_fwd, or NULL (rowsum(dO * O)
 *             is then taken on the bf16 o alone).
 * lse         from prism_attn_fwd.
 * row_ptr/col_idx (query-major) drive dQ; t_row_ptr/t_col_idx (key-major)
 *             drive dK and dV, so no float atomics are used and results are
 *             bitwise reproducible.
 * dq, dk, dv  THW bf16 (out).
 * ws, ws_bytes  workspace (size query as in prism_select_blocks).
 */
int prism_attn_bwd(const prism_problem *prob, const prism_params *par, const prism_bf16 *qp, const prism_bf16 *kp,
                   const prism_bf16 *vp, const prism_bf16 *o, const prism_bf16 *o_lo, const prism_bf16 *dout,
                   const float *lse, const int32_t *perm, const int32_t *blk_start, const int32_t *n_blocks,
                   const int32_t *row_ptr, const int32_t *col_idx, const int32_t *t_row_ptr, const int32_t *t_col_idx, prism_bf16 *dq,
                   prism_bf16 *dk, prism_bf16 *dv, void *ws, size_t *ws_bytes, prism_stream stream);

/*
 * prism_infer_fwd -- the whole forward layer for inference in one call:
 * zone statistics, shapes, permutation, block selection (query-major index
 * only) and sparse attention ([pt/M1]-[pt/M3]), output scattered back to THW
 * ([blog/4]: inference reuses the dynamic sparse logic to save memory).
 * Nothing is kept for a backward pass: no LSE, no key-major index.
 *
 * q, k, v  THW bf16 inputs; a as in prism_zone_stats (NULL = no audio).
 * o        THW bf16 (out).  o may be the same buffer as q, k or v (in place,
 *          element for element); any other overlap is undefined.
 * ws, ws_bytes  workspace (with ws == NULL only the size is stored).  Heads
 *          are processed in passes of par->pass_heads heads (0: enough for
 *          the attention grid to fill the chip, ceil(4096 / (N/64)); at most
 *          all of them) whose intermediates share one workspace; inside a pass
 *          the permuted V rows reuse the memory of the selection scratch.
 *          The block index is sized for the most blocks a row can select
 *          (every block with top_p = 1 and no cap; else max(top_k,
 *          floor(cap N) / 64) blocks), so the call never returns
 *          PRISM_ECAPACITY.
 * Results equal those of prism_zone_stats .. prism_attn_fwd on the same
 * inputs bit for bit.  Synchronises the stream once per pass.
 */
int prism_infer_fwd(const prism_problem *prob, const prism_params *par, const prism_bf16 *q, const prism_bf16 *k,
                    const prism_bf16 *v, const float *a, prism_bf16 *o, void *ws, size_t *ws_bytes,
                    prism_stream stream);

/*
 * prism_dense_attn_fwd / prism_dense_attn_bwd -- full softmax attention over
 * all N tokens (the quadratic cost the method removes), on the same kernels
 * with every key tile selected; the baseline the sparse path is timed
 * against.  THW in and out; lse float [heads][N] in THW order.
 */
int prism_dense_attn_fwd(const prism_problem *prob, const prism_params *par, const prism_bf16 *q,
                         const prism_bf16 *k, const prism_bf16 *v, prism_bf16 *o, float *lse, void *ws,
                         size_t *ws_bytes, prism_stream stream);
int prism_dense_attn_bwd(const prism_problem *prob, const prism_params *par, const prism_bf16 *q,
                         const prism_bf16 *k, const prism_bf16 *v, const prism_bf16 *o, const prism_bf16 *dout,
                         const float *lse, prism_bf16 *dq, prism_bf16 *dk, prism_bf16 *dv, void *ws,
                         size_t *ws_bytes, prism_stream stream);

/*
 * prism_a2v_norms -- the audio guidance map a_n = |h-hat_n|_2 of every video
 * token ([pt/M1], second paragraph: norms of the audio-to-video
 * cross-attention output, cached for the next layer's prism_zone_stats).
 *
 * h_hat        bf16 [n_tokens] x [channels] (row n at h_hat + n * token_stride),
 *              THW token order; 16-byte aligned.
 * n_tokens     rows, 0 <= n_tokens <= INT32_MAX (0 launches nothing).
 * channels     values per row, a positive multiple of 8.
 * token_stride element stride between rows, a multiple of 8, >= channels.
 * a            float [n_tokens] (out): the norm, from a float64 sum of the
 *              (exact) squares, rounded once to float32.
 * Returns PRISM_EINVAL for a NULL or misaligned pointer or a bad size; reads
 * h_hat once (HBM-bound).  Asynchronous on `stream`.
 */
int prism_a2v_norms(const prism_bf16 *h_hat, int64_t n_tokens, int32_t channels, int64_t token_stride, float *a,
                    prism_stream stream);

/*
 * prism_check_index -- validate a block index held in HOST memory, before it
 * is passed to prism_attn_fwd / prism_attn_bwd (which trust the index's
 * contents).  The rules are those every index of the method satisfies
 * ([pt/M2]: each 8x8x8 zone is cut into equal blocks of 64, 128 or 256
 * tokens; [pt/M3]: every query block attends to a non-empty set S_i), in the
 * layout prism_plan_shapes and prism_select_blocks write:
 *  - n_blocks[h] in [N/256, N/64];
 *  - blk_start[h]: starts at 0; every block 1, 2 or 4 tiles of 64 tokens,
 *    aligned to its size and inside one 8-tile zone; entry n_blocks and
 *    every later one equal N/64;
 *  - perm[h] (optional, NULL: not checked): a bijection of [0, N);
 *  - row_ptr/col_idx: offsets counted over all heads (head h starts where
 *    head h-1 ends, head 0 at 0), at most n_idx entries, entries past
 *    n_blocks repeating the head's end; every row non-empty, strictly
 *    ascending key blocks below n_blocks;
 *  - t_row_ptr/t_col_idx (optional, both NULL: not checked): the same
 *    layout (lists may be empty), and exactly the transpose of the
 *    query-major lists.
 * bad  HOST int64 [2] (out, optional): head and item of the first violation
 *      (item: block or row b for blk_start and the query-major lists, token
 *      position for perm, N/64 + 1 + b for key-major list b; -1 for n_blocks).
 * All pointers are HOST pointers; the call touches no device.  Returns
 * PRISM_OK, PRISM_EINDEX at the first violation, PRISM_EGRID or PRISM_EINVAL
 * for bad arguments.
 */
int prism_check_index(const prism_problem *prob, const int32_t *perm, const int32_t *blk_start, const int32_t *n_blocks,
                      const int32_t *row_ptr, const int32_t *col_idx, const int32_t *t_row_ptr,
                      const int32_t *t_col_idx, int64_t n_idx, int64_t *bad);

/*
 * prism_sclk_probe -- the shader clock the chip holds under a sustained
 * matrix-core load (a measurement aid for stating MFMA rates against the
 * peak at the clock actually run, not a step of the method).  Runs about
 * 8 ms of independent bf16 MFMAs at two waves per SIMD on every CU and
 * compares the shader-clock counter with the constant 100 MHz counter.
 * ghz  HOST double (out): the clock in GHz.
 * Synchronises `stream`.  Uses a 64 KiB array in the library's module
 * memory (allocates nothing); calls that overlap on one GPU race.  Returns
 * PRISM_EINVAL for a NULL pointer, PRISM_EHIP for a runtime error.
 */
int prism_sclk_probe(double *ghz, prism_stream stream);

/* Human-readable text of a status code (static storage). */
const char *prism_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* PRISM_H */

/*
 * veda.h - C ABI of the Veda tile-sparse self-attention forward for AMD
 * MI355X (gfx950).
 *
 * Method: "Veda: Scalable Video Diffusion via Distilled Sparse Attention"
 * (project page veda-sparse.github.io). One attention layer is five calls:
 *
 *   veda_tile_permute      x3  raster Q/K/V -> head-specific 128-token tiles
 *   veda_trippool_score        TripPool stats -> head-specific projections -> tile scores
 *   veda_topk_mask             head-aware Top-k per query tile -> index lists (+ bitmask)
 *   veda_sparse_attn_fwd       flash-attention forward over the selected K/V tiles only
 *   veda_tile_unpermute        tiled O -> raster O
 *
 * The same layer in fewer passes over HBM, with identical results:
 *   veda_tile_permute_stats    x2  raster Q/K -> tiles and each tile's TripPool stats in one pass
 *   veda_trippool_project_score    stats -> head-specific projections (-> tile scores)
 *   veda_score_topk            tile scores and Top-k in one pass, from the projections (no score
 *                              matrix; or veda_topk_mask of the scores the call above writes)
 *   veda_sparse_attn_fwd_raster    attention that writes raster O itself (no unpermute pass)
 *   (with veda_tile_permute of V in between)
 * and with Q never tiled: veda_tile_permute_stats of Q with no tiled output (statistics
 * only), then veda_sparse_attn_fwd_raster_io, which also reads Q in raster order.
 *
 * Dense attention, the baseline the tile-sparse layer is measured against:
 *   veda_dense_attn_fwd        every key tile kept, no index list (also veda_dense_attn_fwd_raster)
 *
 * More calls measure the mask against the method's own target:
 *   veda_teacher_tile_max      max-pooled dense attention per (query tile, key tile); its
 *                              veda_topk_mask is the oracle tile mask
 *   veda_avgpool_score         average-pooling tile scores, the pages' baseline mask
 *   veda_tile_scores_mfma      the estimator's scores on the matrix cores (within rounding of the
 *                              ordered scores, not bit-identical)
 *   veda_mask_overlap          common kept tiles of two masks
 *   veda_tile_recall           tile recall of a mask against the oracle mask
 *   veda_head_sq_error         squared output error per head (objective of the head-aware tile search)
 *   veda_candidate_tiles       the tile shapes the search tries (host only)
 *   veda_tile_search_select    per head, the candidate tiling with the smallest error
 *   veda_k_from_keep           k_hd from a keep fraction (host only)
 *
 * Distilling the estimator's projections toward the teacher:
 *   veda_distill_kl            KL(teacher row || softmax(scores)) per query tile and its gradient
 *   veda_distill_mean_kl       the mean KL over the query tiles (the reported loss)
 *   veda_distill_grad          that gradient back to W_q and W_k
 *   veda_adam_step             one Adam update of fp32 master weights (+ their bf16 copy)
 *
 * Conventions shared by every call
 * --------------------------------
 * Tensors are DEVICE pointers allocated and owned by the caller; the library
 * never allocates, frees or caches device memory and keeps no state between
 * calls (re-entrant, thread-safe). The one exception is
 * veda_sparse_attn_fwd_raster_io_noalloc, whose 64-byte work queue is a static
 * device array of the library, shared by every call on a device. Small arrays marked "host" are read during
 * the call only. `stream` is a hipStream_t (NULL = the default stream); every
 * call only enqueues work on it and never synchronises, so results are
 * visible in stream order. Inputs are read-only; outputs must not overlap
 * inputs or each other.
 *
 * Geometry. The latent grid is (T, H, W); the raster token index is
 * n = (t*H + y)*W + x. Head hd uses tile (pt, ph, pw) with pt*ph*pw = 128
 * (so each edge is a power of two). Each axis is padded up to a multiple of
 * the tile edge, giving nT_hd = ceil(T/pt)*ceil(H/ph)*ceil(W/pw) tiles;
 * nT_max is the largest nT_hd over heads. Tiles are numbered in raster order
 * of their box coordinates and the 128 slots of a tile in raster order of
 * the offsets (t%pt, y%ph, x%pw). A slot no real token maps to is a pad slot.
 *
 * Layouts (row-major, contiguous unless a stride is given):
 *   raster x        [B, N, heads, d] bf16 with element strides veda_raster_strides (channel stride 1)
 *   tiled x         [B, heads, nT_max, 128, d] bf16 (token-major), or
 *                   [B, heads, nT_max, d, 128] bf16 (channel-major: each tile transposed).
 *                   The attention calls take V channel-major: its rows are the rows of V^T, the
 *                   operand the PV matrix product reads, 8 consecutive keys of one channel per
 *                   16-byte read. (Token-major V read through the LDS transpose reads measured
 *                   9% slower.)
 *   stats           [B, heads, nT_max, 3d] bf16, [avg | max | min]
 *   features        [B, heads, nT_max, r] bf16
 *   W_q, W_k        [heads, 3d, r] bf16 (features = stats @ W)
 *   scores          [B, heads, nT_max, nT_max] fp32
 *   idx             [B, heads, nT_max, k_max] int32
 *   bitmask         [B, heads, nT_max, ceil(nT_max/32)] uint32
 *   lse             [B, heads, nT_max, 128] fp32
 *
 * Defined outputs: every output byte is written. Pad slots of tiled tensors
 * hold 0; tiles with index >= nT_hd hold 0 (tiled, stats, features), -inf
 * (scores and lse) or -1 (idx) and 0 (bitmask); scores outside the head's
 * nT_hd x nT_hd block are -inf; idx entries past k_hd are -1.
 *
 * Values: device data is never inspected, and inputs are expected finite.
 * A NaN score orders by its bit pattern (above every finite score with the
 * sign bit clear, below with it set), so index lists stay ascending, in
 * range and k_hd long; a NaN or inf in Q, K, V or W reaches the outputs
 * computed from it.
 *
 * Errors: every call returns VEDA_OK (0) or a negative status. All argument
 * checks run on the host BEFORE anything is enqueued, so a call that fails
 * them writes nothing. Checks: null pointers; B, heads or a grid edge <= 0;
 * heads > VEDA_MAX_HEADS; d not 64 or 128; r not 32 or 64; a tile whose
 * volume is not 128; nT_max > VEDA_MAX_TILES; k_hd outside [1, nT_hd] or
 * above k_max; a tensor pointer not 16-byte aligned or a raster stride not a
 * multiple of 8 elements; the current device not gfx950. A failed launch
 * returns VEDA_ERR_LAUNCH. Nothing throws or aborts across this ABI.
 */
#ifndef VEDA_H_
#define VEDA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VEDA_TILE_TOKENS 128
#define VEDA_MAX_HEADS 128
#define VEDA_MAX_TILES 8192
/* Size of the work-queue workspace the attention calls may take. */
#define VEDA_ATTN_QUEUE_BYTES 64

/* Layout of a tiled tensor: token-major [.., 128, d] or channel-major [.., d, 128]. */
enum { VEDA_TILED_TOKEN_MAJOR = 0, VEDA_TILED_CHANNEL_MAJOR = 1 };

enum {
  VEDA_OK = 0,
  VEDA_ERR_NULL = -1,    /* a required pointer is NULL */
  VEDA_ERR_SHAPE = -2,   /* B, heads, grid, d, r or a size limit out of range */
  VEDA_ERR_TILE = -3,    /* a head's tile volume is not 128 */
  VEDA_ERR_K = -4,       /* k_hd outside [1, nT_hd] or above k_max */
  VEDA_ERR_ALIGN = -5,   /* a pointer not 16-byte aligned, or a stride not a multiple of 8 */
  VEDA_ERR_DEVICE = -6,  /* no HIP device, or the current device is not gfx950 */
  VEDA_ERR_LAUNCH = -7   /* a kernel launch failed */
};

typedef struct { int32_t T, H, W; } veda_grid;
typedef struct { int32_t pt, ph, pw; } veda_tile;

typedef struct {
  int32_t B;                   /* batch, 1..65535 (an empty batch is VEDA_ERR_SHAPE) */
  int32_t n_heads;             /* attention heads, 1..VEDA_MAX_HEADS */
  int32_t head_dim;            /* d: 64 or 128 */
  veda_grid grid;              /* latent grid (T, H, W), each extent >= 1 */
  const veda_tile* head_tile;  /* host array [n_heads]: tile shape of each head */
} veda_geom;

/* Element strides of a raster tensor [B, N, heads, d]; the channel stride is 1. */
typedef struct { int64_t b, n, h; } veda_raster_strides;

/* Text of a status code (static storage). */
const char* veda_status_str(int status);

/* Tiles of head `head` (host only, no device work): nT_hd >= 1, or a negative status. */
int veda_num_tiles(const veda_geom* g, int32_t head);

/* Largest tile count over heads (host only): nT_max >= 1, or a negative status. */
int veda_max_tiles(const veda_geom* g);

/*
 * Head-conditioned re-tiling of a raster tensor (Veda page, "Architecture",
 * Principle 02 "Head-Conditioned Tile Geometry": per-head tile shapes
 * (p_t, p_h, p_w); "Head-Aware Tile Search": p_t*p_h*p_w = B = 128).
 *   x_raster  in   raster bf16 tensor, strides `s` (elements)
 *   x_tiled   out  tiled bf16 in `layout`: VEDA_TILED_TOKEN_MAJOR [B, heads, nT_max, 128, d] or
 *                  VEDA_TILED_CHANNEL_MAJOR [B, heads, nT_max, d, 128] (the layout the attention
 *                  call takes V in); pad slots and tiles >= nT_hd are 0
 *   layout    in   VEDA_TILED_TOKEN_MAJOR or VEDA_TILED_CHANNEL_MAJOR (else VEDA_ERR_SHAPE)
 */
int veda_tile_permute(const veda_geom* g, const void* x_raster, veda_raster_strides s,
                      void* x_tiled, int32_t layout, void* stream);

/*
 * Token-major re-tiling of Q or K fused with the TripPool statistics of each
 * tile (Veda page, "Architecture", Principle 02 "Head-Conditioned Tile
 * Geometry"; "Attention Structure Distillation", Estimator: average, maximum
 * and minimum per tile). One pass over the raster tensor writes both outputs:
 *   x_raster  in   raster bf16 tensor, strides `s` (elements)
 *   x_tiled   out  bf16 [B, heads, nT_max, 128, d], exactly as veda_tile_permute with
 *                  VEDA_TILED_TOKEN_MAJOR writes it; may be NULL: then only the statistics are
 *                  computed, in a pass that only reads x_raster (the layer does this for Q,
 *                  which veda_sparse_attn_fwd_raster_io reads in raster order)
 *   stats     out  bf16 [B, heads, nT_max, 3d], exactly the stats_q (or stats_k) that
 *                  veda_trippool_score computes from x_tiled (0 for tiles >= nT_hd)
 * Errors: a null x_raster or stats (VEDA_ERR_NULL), a pointer not 16-byte aligned or a stride
 * not a multiple of 8 (VEDA_ERR_ALIGN), and the geometry checks of every call.
 */
int veda_tile_permute_stats(const veda_geom* g, const void* x_raster, veda_raster_strides s,
                            void* x_tiled, void* stats, void* stream);

/*
 * TripPool estimator (Veda page, "Attention Structure Distillation",
 * Estimator: average, maximum and minimum per tile, then head-specific Q/K
 * projections score each query-tile x key-tile pair; "Theoretical
 * Rationale" 2 "Tile Statistics").
 *   q_tiled, k_tiled  in   tiled bf16 Q and K
 *   w_q, w_k          in   bf16 [heads, 3d, rank]
 *   rank              in   r: 32 or 64
 *   stats_q, stats_k  out  bf16 [B, heads, nT_max, 3d]: avg (fp32 sum in slot order over real
 *                          tokens from +0, correctly rounded divide, round-to-nearest-even to
 *                          bf16), max and min (exact; -0 orders below +0)
 *   feat_q, feat_k    out  bf16 [B, heads, nT_max, rank]: stats @ W, fp32 accumulated one
 *                          channel at a time in ascending order from +0, then rounded to bf16
 *   scores            out  fp32 [B, heads, nT_max, nT_max]: feat_q . feat_k, fp32 accumulated
 *                          in ascending channel order from +0; -inf outside the head's block
 * The fixed accumulation order makes every output reproducible bit for bit.
 */
int veda_trippool_score(const veda_geom* g, const void* q_tiled, const void* k_tiled,
                        const void* w_q, const void* w_k, int32_t rank,
                        void* stats_q, void* stats_k, void* feat_q, void* feat_k,
                        float* scores, void* stream);

/*
 * The projection and scoring half of veda_trippool_score, from statistics
 * already computed (by veda_tile_permute_stats of Q and of K). Same page and
 * passage as veda_trippool_score.
 *   stats_q, stats_k  in   bf16 [B, heads, nT_max, 3d], [avg | max | min]
 *   w_q, w_k          in   bf16 [heads, 3d, rank]
 *   rank              in   r: 32 or 64 (else VEDA_ERR_SHAPE)
 *   feat_q, feat_k    out  bf16 [B, heads, nT_max, rank], as veda_trippool_score
 *   scores            out  fp32 [B, heads, nT_max, nT_max], as veda_trippool_score; may be NULL,
 *                          and then only the features are computed (veda_score_topk takes the
 *                          mask from them without a score matrix)
 * Given the statistics veda_trippool_score would compute, the outputs are
 * identical to its outputs, bit for bit.
 */
int veda_trippool_project_score(const veda_geom* g, const void* stats_q, const void* stats_k,
                                const void* w_q, const void* w_k, int32_t rank,
                                void* feat_q, void* feat_k, float* scores, void* stream);

/*
 * Tile scores as the small bf16 GEMM the estimator is (Veda page, "Attention Structure Distillation",
 * Estimator: the scores of every (query tile, key tile) pair are the products of the head-specific
 * projections), computed on the matrix cores: S[b, hd, i, j] = sum over c of feat_q[i, c] * feat_k[j, c]
 * with bf16 MFMA instructions accumulating in fp32 in the hardware's own order.
 *   feat_q, feat_k    in   bf16 [B, heads, nT_max, rank], as veda_trippool_project_score writes them
 *   rank              in   32 or 64 (else VEDA_ERR_SHAPE)
 *   scores            out  fp32 [B, heads, nT_max, nT_max]; -inf outside the head's nT_hd x nT_hd block
 * Each product of two bf16 values is exact in fp32, so each score differs from the ordered sum that
 * veda_trippool_project_score computes by at most the rounding of an fp32 sum of rank terms:
 * |S_mfma - S_ordered| <= 2 * gamma_rank * sum over c of |feat_q[i, c] * feat_k[j, c]|, with
 * gamma_n = n u / (1 - n u), u = 2^-24. The two are often bit-identical but not always, so a
 * veda_topk_mask of these scores can differ from the ordered path's where two key tiles are that
 * close. The layer's route uses the ordered path, whose masks are reproducible bit for bit; this call
 * is the faster alternative for callers that accept near-tie differences.
 */
int veda_tile_scores_mfma(const veda_geom* g, const void* feat_q, const void* feat_k, int32_t rank,
                          float* scores, void* stream);

/*
 * Average-pooling tile scores, the baseline mask the pages compare Veda's against at the same budget
 * (Veda page, "Empirical Study", 02 "Controlled Mask Intervention"): the dot product of the tile
 * means alone, over all d channels, with no projection. veda_topk_mask of these scores gives the
 * average-pooling mask; veda_mask_overlap against the teacher's oracle mask gives its tile recall.
 *   stats_q, stats_k  in   bf16 [B, heads, nT_max, 3d] (veda_tile_permute_stats or
 *                          veda_trippool_score); only the avg block (channels 0..d-1) is read
 *   scores            out  fp32 [B, heads, nT_max, nT_max]: sum over c < d of avg_q[i, c] * avg_k[j, c],
 *                          fp32 accumulated in ascending c from +0; -inf outside the head's block
 * Errors: null or unaligned pointers, and the geometry checks of every call.
 */
int veda_avgpool_score(const veda_geom* g, const void* stats_q, const void* stats_k, float* scores,
                       void* stream);

/*
 * Head-aware Top-k tile mask (Veda page, "Attention Structure Distillation",
 * Execution: Top-k per query tile gives the binary tile mask). For every
 * (b, hd, query tile) the k_hd largest scores among key tiles 0..nT_hd-1;
 * equal scores go to the lower tile index and -0 equals +0.
 *   scores      in   fp32 [B, heads, nT_max, nT_max] (finite within each head's block)
 *   k_per_head  in   host int32 [heads]: k_hd, 1 <= k_hd <= nT_hd, k_hd <= k_max
 *   k_max       in   row length of idx
 *   idx         out  int32 [B, heads, nT_max, k_max]: kept tiles ascending, then -1
 *   bitmask     out  uint32 [B, heads, nT_max, ceil(nT_max/32)], bit j%32 of word j/32; may be NULL
 */
int veda_topk_mask(const veda_geom* g, const float* scores, const int32_t* k_per_head,
                   int32_t k_max, int32_t* idx, uint32_t* bitmask, void* stream);

/*
 * Tile scores and head-aware Top-k in one pass (Veda page, "Attention Structure Distillation",
 * Estimator and Execution: the projections' products score the tile pairs, and Top-k per query
 * tile of those scores is the tile mask). The scores of a group of query tiles are held on chip
 * and selected there; no score matrix is written or read.
 *   feat_q, feat_k    in   bf16 [B, heads, nT_max, rank], as veda_trippool_project_score writes them
 *   rank              in   32 or 64 (else VEDA_ERR_SHAPE)
 *   k_per_head, k_max, idx, bitmask   as veda_topk_mask
 * The scores are those veda_trippool_project_score writes (fp32 FMA over the channels in ascending
 * order from +0), so idx and bitmask are, bit for bit, what veda_topk_mask makes of them.
 * nT_max must not exceed 2048 (else VEDA_ERR_SHAPE; use the two calls).
 */
int veda_score_topk(const veda_geom* g, const void* feat_q, const void* feat_k, int32_t rank,
                    const int32_t* k_per_head, int32_t k_max, int32_t* idx, uint32_t* bitmask,
                    void* stream);

/*
 * Tile-skipping attention forward (Veda page, "Attention Structure
 * Distillation", Execution: the kernel fetches only the selected K/V tiles;
 * "Principle 03" Tile-Sparse Kernel; "Theoretical Rationale" 1 "Softmax
 * Geometry": each query row is a softmax over the kept keys, i.e. the dense
 * probabilities renormalised by Z / Z_hat, with log-sum-exp LSE).
 * Query token i of tile tq attends to the real (non-pad) keys of the tiles
 * idx[b, hd, tq, 0..k_hd-1]; logits are scale * q.k; bf16 MFMA products with
 * fp32 accumulation and an fp32 online softmax.
 *   q_tiled, k_tiled           in   tiled bf16, token-major [B, heads, nT_max, 128, d]
 *   v_tiled                    in   tiled bf16, channel-major [B, heads, nT_max, d, 128]
 *   idx                        in   int32 [B, heads, nT_max, k_max] from veda_topk_mask
 *                                   (entries 0..k_hd-1 must lie in [0, nT_hd))
 *   k_per_head                 in   host int32 [heads]
 *   softmax_scale              in   logit scale; <= 0 selects 1/sqrt(d)
 *   o_tiled                    out  tiled bf16 O; tiles >= nT_hd are 0; pad query slots hold the
 *                                   output of a zero query
 *   lse                        out  fp32 [B, heads, nT_max, 128], natural log of the softmax
 *                                   denominator of the scaled logits; -inf for tiles >= nT_hd; may be NULL
 *   work_queue                 tmp  device workspace of VEDA_ATTN_QUEUE_BYTES (16-byte aligned), or
 *                                   NULL. With it, query tiles are handed out at run time so that
 *                                   XCDs running at different clocks finish together; the call
 *                                   first clears it with a kernel on `stream` (no memset). Calls
 *                                   that may run at the same time need separate workspaces. With
 *                                   NULL, or when B * heads * nT_max < 1024 (nothing to balance),
 *                                   every XCD gets a fixed share and the workspace is not touched.
 *                                   The outputs are the same bytes either way. With a workspace,
 *                                   B * heads * nT_max must not exceed 2^28 (else VEDA_ERR_SHAPE).
 */
int veda_sparse_attn_fwd(const veda_geom* g, const void* q_tiled, const void* k_tiled,
                         const void* v_tiled, const int32_t* idx, const int32_t* k_per_head,
                         int32_t k_max, float softmax_scale, void* o_tiled, float* lse,
                         int32_t* work_queue, void* stream);

/*
 * The same attention forward writing O straight into raster order, which
 * spares the tile unpermute pass (Veda page, same passages; the raster O is
 * the inverse of the head-conditioned re-tiling, "Architecture", Principle 02).
 * Arguments as veda_sparse_attn_fwd, except:
 *   o_raster  out  raster bf16 [B, N, heads, d] with element strides `s` (channel stride 1): the
 *                  row of every real token of every head is written; nothing else is touched
 *   s         in   strides of o_raster (elements; multiples of 8, else VEDA_ERR_ALIGN)
 *   lse       out  as veda_sparse_attn_fwd for real query slots; -inf for pad query slots, which
 *                  have no raster row (a group of 32 pad slots is not computed at all)
 * For the same inputs, o_raster holds exactly the bytes veda_tile_unpermute of veda_sparse_attn_fwd's
 * o_tiled would give, and lse matches veda_sparse_attn_fwd's on every real query slot.
 */
int veda_sparse_attn_fwd_raster(const veda_geom* g, const void* q_tiled, const void* k_tiled,
                                const void* v_tiled, const int32_t* idx, const int32_t* k_per_head,
                                int32_t k_max, float softmax_scale, void* o_raster,
                                veda_raster_strides s, float* lse, int32_t* work_queue, void* stream);

/*
 * The same attention reading Q in raster order as well, so no tiled copy of Q
 * is needed (the re-tiling of Q, "Architecture", Principle 02, happens in the
 * kernel's own loads). Arguments as veda_sparse_attn_fwd_raster, except:
 *   q_raster  in   raster bf16 Q [B, N, heads, d] with element strides `sq` (channel stride 1,
 *                  multiples of 8); each query slot reads its token's row, and a pad slot a zero
 *                  query, exactly what tiled Q holds
 *   o_raster  out  as o_raster of veda_sparse_attn_fwd_raster, with strides `so`
 * For the same inputs the outputs are the bytes veda_sparse_attn_fwd_raster gives with the
 * tiled Q that veda_tile_permute makes of q_raster.
 */
int veda_sparse_attn_fwd_raster_io(const veda_geom* g, const void* q_raster, veda_raster_strides sq,
                                   const void* k_tiled, const void* v_tiled, const int32_t* idx,
                                   const int32_t* k_per_head, int32_t k_max, float softmax_scale,
                                   void* o_raster, veda_raster_strides so, float* lse,
                                   int32_t* work_queue, void* stream);

/*
 * Dense attention forward: every key tile kept (Veda page, "Scaling Law in Practice": the dense
 * FlashAttention baseline the tile-sparse layer is timed against; "Attention Structure Distillation",
 * Teacher: the full attention whose LSE the teacher needs). The same kernel as the tile-sparse
 * forward with the kept tiles of every query tile being key tiles 0..nT_hd-1 in order, so no index
 * list exists or is read; the outputs are the bytes veda_sparse_attn_fwd gives with idx[.., j] = j
 * and k_hd = nT_hd.
 *   q_tiled, k_tiled, v_tiled, softmax_scale, lse, work_queue   as veda_sparse_attn_fwd
 *   o_tiled                                                     out  tiled bf16 O, as veda_sparse_attn_fwd
 */
int veda_dense_attn_fwd(const veda_geom* g, const void* q_tiled, const void* k_tiled, const void* v_tiled,
                        float softmax_scale, void* o_tiled, float* lse, int32_t* work_queue, void* stream);

/*
 * Dense attention writing raster O (as veda_sparse_attn_fwd_raster does for the tile-sparse call).
 *   o_raster, s   out  raster bf16 O with element strides `s`; lse as veda_sparse_attn_fwd_raster
 */
int veda_dense_attn_fwd_raster(const veda_geom* g, const void* q_tiled, const void* k_tiled, const void* v_tiled,
                               float softmax_scale, void* o_raster, veda_raster_strides s, float* lse,
                               int32_t* work_queue, void* stream);

/*
 * Allocation-free form of veda_sparse_attn_fwd_raster_io, for callers that cannot allocate device
 * memory or bring a workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). Arguments and outputs are those of veda_sparse_attn_fwd_raster_io with a work
 * queue, minus work_queue: the queue lives in a static 64-byte device array of the library (one per
 * device, held until the process ends), whose address is looked up once per device. The call itself
 * allocates nothing; it clears the queue with a kernel on `stream` before each launch (as with a
 * caller's workspace), so the outputs are the bytes veda_sparse_attn_fwd_raster_io gives.
 * Limit: B * heads * nT_max <= 2^28 work items (else VEDA_ERR_SHAPE), as for a workspace.
 * Every call on one device shares that device's array: calls that may overlap in time on one device
 * (other streams, other threads) race on it; give those veda_sparse_attn_fwd_raster_io with
 * workspaces of their own. A failed symbol lookup returns VEDA_ERR_DEVICE.
 */
int veda_sparse_attn_fwd_raster_io_noalloc(const veda_geom* g, const void* q_raster, veda_raster_strides sq,
                                           const void* k_tiled, const void* v_tiled, const int32_t* idx,
                                           const int32_t* k_per_head, int32_t k_max, float softmax_scale,
                                           void* o_raster, veda_raster_strides so, float* lse, void* stream);

/*
 * Inverse re-tiling: raster x[b, n, hd, :] = tiled x at the slot of token n
 * (the inverse of veda_tile_permute; pad slots are dropped).
 *   x_tiled   in   tiled bf16 [B, heads, nT_max, 128, d]
 *   x_raster  out  raster bf16 tensor, strides `s`; every (b, n, hd, c) element is written
 */
int veda_tile_unpermute(const veda_geom* g, const void* x_tiled, void* x_raster,
                        veda_raster_strides s, void* stream);

/*
 * Tile-level teacher (Veda page, "Attention Structure Distillation", Teacher: max-pooled full
 * attention as tile-level supervision; Principle 01; "Empirical Study" 02: the oracle mask keeps the
 * highest-response key tiles of each query tile):
 *   T[b, hd, tq, j] = max over real queries i of tile tq and real keys m of tile j of
 *                     exp(scale * q_i . k_m - lse_i),
 * the largest dense softmax probability between the two tiles (bf16 MFMA products, fp32 accumulation).
 *   q_tiled, k_tiled  in   tiled bf16, token-major [B, heads, nT_max, 128, d]
 *   lse_dense         in   fp32 [B, heads, nT_max, 128]: the lse output of veda_sparse_attn_fwd run with
 *                          every key tile kept (k_hd = nT_hd, idx[..., j] = j), same softmax_scale
 *   softmax_scale     in   <= 0 selects 1/sqrt(d)
 *   teacher           out  fp32 [B, heads, nT_max, nT_max], values in (0, 1]; -inf outside the head's
 *                          nT_hd x nT_hd block. veda_topk_mask(teacher) gives the oracle tile mask.
 *   work_queue        tmp  as veda_sparse_attn_fwd (query tiles handed out at run time, or NULL)
 */
int veda_teacher_tile_max(const veda_geom* g, const void* q_tiled, const void* k_tiled, const float* lse_dense,
                          float softmax_scale, float* teacher, int32_t* work_queue, void* stream);

/*
 * Overlap of two tile masks (tile recall of a mask against an oracle mask is
 * counts / (k_hd * nT_hd)).
 *   bitmask_a, bitmask_b  in   uint32 [B, heads, nT_max, ceil(nT_max/32)] from veda_topk_mask
 *   counts                out  uint64 [B, heads]: sum over the head's query tiles of popcount(a & b)
 */
int veda_mask_overlap(const veda_geom* g, const uint32_t* bitmask_a, const uint32_t* bitmask_b, uint64_t* counts,
                      void* stream);

/*
 * Tile recall of a mask against the oracle mask (Veda page, "Empirical Study", 02 "Controlled Mask
 * Intervention": the share of the oracle mask's kept tiles that a mask also keeps):
 *   recall[b, hd] = (sum over the head's query tiles of popcount(mask & oracle)) / (k_hd * nT_hd)
 *   bitmask, bitmask_oracle  in   uint32 [B, heads, nT_max, ceil(nT_max/32)] from veda_topk_mask
 *   k_per_head               in   host int32 [heads]: the oracle mask's k_hd (1 <= k_hd <= nT_hd)
 *   counts                   out  uint64 [B, heads], the numerators (as veda_mask_overlap); may be NULL
 *   recall                   out  fp64 [B, heads]
 */
int veda_tile_recall(const veda_geom* g, const uint32_t* bitmask, const uint32_t* bitmask_oracle,
                     const int32_t* k_per_head, uint64_t* counts, double* recall, void* stream);

/*
 * Squared error per (batch, head) between two raster tensors (Veda page, "Head-Aware Tile Search":
 * each head takes the tiling that minimises ||O_full - O_sparse||_F^2 on calibration samples):
 *   err[b, hd] = sum over tokens n and channels c of (a[b, n, hd, c] - b[b, n, hd, c])^2,
 * summed in fp64 in a fixed order (deterministic).
 *   a_raster, b_raster  in   raster bf16 tensors [B, N, heads, d], strides sa, sb (elements)
 *   err                 out  fp64 [B, heads]
 */
int veda_head_sq_error(const veda_geom* g, const void* a_raster, veda_raster_strides sa, const void* b_raster,
                       veda_raster_strides sb, double* err, void* stream);

/*
 * The head-aware tile search's choice (Veda page, "Head-Aware Tile Search": each head takes the
 * candidate tiling that minimises ||O_full - O_sparse||_F^2 on calibration samples):
 *   err_sum[c, hd] = sum over b (ascending) of err[c, b, hd] in fp64;
 *   best[hd] = the c with the smallest err_sum[c, hd]; equal sums keep the lower c, and a NaN sum is
 *              never taken over a number.
 *   err      in   fp64 [n_candidates, B, heads] (veda_head_sq_error of each candidate's layer)
 *   err_sum  out  fp64 [n_candidates, heads]; may be NULL
 *   best     out  int32 [heads]
 * Errors: n_candidates, B or heads <= 0, heads > VEDA_MAX_HEADS or B > 65535 (VEDA_ERR_SHAPE).
 */
int veda_tile_search_select(int32_t n_candidates, int32_t B, int32_t heads, const double* err, double* err_sum,
                            int32_t* best, void* stream);

/*
 * Candidates of the head-aware tile search (host only; Veda page, "Head-Aware Tile Search": tile
 * shapes whose three edges multiply to the 128-token budget): every (pt, ph, pw) of powers of two
 * with pt*ph*pw = 128, each edge at most the grid's, and at most VEDA_MAX_TILES tiles, in order of
 * increasing pt, then ph. There are at most 36.
 *   tiles     out  host array of `capacity` entries
 * Returns the number written, or VEDA_ERR_NULL, or VEDA_ERR_SHAPE (a grid edge <= 0, or more
 * candidates than `capacity`).
 */
int veda_candidate_tiles(veda_grid grid, veda_tile* tiles, int32_t capacity);

/*
 * k from a keep fraction (host only, no device work; reading of "top-k = p% of key tiles"):
 * k_hd = ceil(keep * nT_hd) with keep = keep_num / keep_den in (0, 1], exactly in integers,
 * clamped to [1, nT_hd]. Returns k_hd, or VEDA_ERR_K for a fraction outside (0, 1] and the
 * geometry errors of every call (VEDA_ERR_SHAPE for a head outside [0, heads)).
 */
int veda_k_from_keep(const veda_geom* g, int32_t head, int64_t keep_num, int64_t keep_den);

/*
 * Distillation objective (Veda page, "Theoretical Rationale" 4, "Distillation Objective": the
 * estimator's soft tile distribution is aligned with the max-pooled full-attention target by a KL
 * divergence before Top-k; Principle 01). Per (b, hd, query tile tq < nT_hd), over key tiles j < nT_hd:
 *   A_tgt = teacher / sum_j teacher,  A_pred = softmax_j(scores),
 *   kl_rows = sum_j A_tgt (log A_tgt - log A_pred),  d_scores = grad_scale * (A_pred - A_tgt).
 *   scores      in   fp32 [B, heads, nT_max, nT_max] (veda_trippool_score)
 *   teacher     in   fp32 [B, heads, nT_max, nT_max] (veda_teacher_tile_max)
 *   grad_scale  in   factor on the gradient (e.g. 1 / number of rows for a mean loss); finite
 *   kl_rows     out  fp32 [B, heads, nT_max]; 0 for query tiles >= nT_hd
 *   d_scores    out  fp32 [B, heads, nT_max, nT_max]; 0 outside the head's block
 * fp32 throughout, fixed summation order.
 */
int veda_distill_kl(const veda_geom* g, const float* scores, const float* teacher, float grad_scale, float* kl_rows,
                    float* d_scores, void* stream);

/*
 * The distillation loss as reported: the mean of kl_rows (veda_distill_kl) over the query tiles
 * that exist, (b, hd, tq < nT_hd), summed in fp64 in a fixed order (reproducible).
 *   kl_rows  in   fp32 [B, heads, nT_max]
 *   mean     out  one fp64 value (8-byte aligned)
 */
int veda_distill_mean_kl(const veda_geom* g, const float* kl_rows, double* mean, void* stream);

/*
 * Gradient of the distillation loss with respect to the head-specific projections, through
 * scores = feat_q . feat_k and feat = stats @ W (the bf16 rounding of feat taken as the identity):
 *   d_feat_q = d_scores @ feat_k,  d_feat_k = d_scores^T @ feat_q   (per b, hd; fp32 [B, heads, nT_max, rank],
 *                                                                   0 for tiles >= nT_hd)
 *   d_w_q = sum_b stats_q^T @ d_feat_q,  d_w_k likewise             (fp32 [heads, 3d, rank])
 *   stats_q, stats_k, feat_q, feat_k  in  bf16, as written by veda_trippool_score with this rank
 * fp32 accumulation in ascending order of the contraction index (reproducible bit for bit).
 */
int veda_distill_grad(const veda_geom* g, int32_t rank, const void* stats_q, const void* stats_k, const void* feat_q,
                      const void* feat_k, const float* d_scores, float* d_feat_q, float* d_feat_k, float* d_w_q,
                      float* d_w_k, void* stream);

/*
 * One Adam step (bias-corrected) on n fp32 master weights, in place:
 *   m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g^2;
 *   w -= lr * (m / (1 - beta1^step)) / (sqrt(v / (1 - beta2^step)) + eps)
 * and, when w_bf16 is not NULL, its bf16 copy (round to nearest even) for veda_trippool_score.
 * step >= 1; 0 <= beta < 1; eps > 0. Error VEDA_ERR_SHAPE otherwise.
 */
int veda_adam_step(int64_t n, float* w_master, const float* grad, float* m, float* v, int32_t step, float lr,
                   float beta1, float beta2, float eps, void* w_bf16, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VEDA_H_ */

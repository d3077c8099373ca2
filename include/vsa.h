/*
 * vsa.h - C ABI of the block-sparse video attention library (libvsa.so).
 *
 * The library computes block-sparse self-attention over the 3D latent token
 * grid (T x H x W) of a video diffusion transformer on AMD Instinct MI355X
 * (gfx950). Tokens are regrouped into tiles, a per-query-tile list of key
 * tiles is built (fixed window / Skiparse-2D pattern, or adaptive top-k /
 * top-p routing over mean-pooled tiles), and a flash-style forward pass
 * visits only the listed key/value tiles, in bf16 or in fp8 e4m3 with one
 * scale per tile.
 *
 * Sources of each operation (titles and sections of the pages that define
 * the method):
 *   - "FPSAttention: Training-Aware FP8 and Sparsity Co-Design for Fast Video
 *     Diffusion", Approach: FP8 quantisation and block sparsity on one shared
 *     3D tile granularity; sliding tile windows.
 *   - "OSP-Next" model card, Model Summary: Skiparse-2D, a fixed strided
 *     sparse pattern applied along H and W, mixed with full attention.
 *   - "Faster Video Diffusion with Trainable Sparse Attention" (VSA),
 *     Research Type row: adaptive selection of key blocks per query block.
 *   - "FVAttn" summary: Top-p routing with a Top-k safety floor over
 *     video-aware blocks, per head.
 *
 * Conventions shared by every call:
 *   - Ownership: every buffer is allocated and owned by the caller. Tensor
 *     arguments are DEVICE pointers; vsa_layout / vsa_layout_info are HOST
 *     structs passed by pointer and only read during the call. The library
 *     allocates nothing and keeps no state between calls.
 *   - Streams: `stream` is a hipStream_t (NULL = the default stream). Calls
 *     only enqueue work on it and never synchronise.
 *   - Errors: every argument check runs on the host before any launch, so a
 *     call that returns an error has written nothing. A failed launch returns
 *     VSA_ERR_HIP. vsa_last_error() gives a thread-local message for the last
 *     failing call on the calling thread.
 *   - Layouts: tensors are dense and row-major in the shapes given below, and
 *     base pointers must be 16-byte aligned.
 *   - Natural order: token n = (t * H + h) * W + w. Tiled order: see
 *     vsa_tile_permute.
 */
#ifndef VSA_H_
#define VSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ----- status codes ------------------------------------------------------- */
typedef enum vsa_status {
  VSA_OK = 0,
  VSA_ERR_INVALID = 1,      /* a null pointer, a bad size or an inconsistent argument */
  VSA_ERR_UNSUPPORTED = 2,  /* valid, but outside what the kernels implement */
  VSA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  VSA_ERR_HIP = 4           /* the HIP runtime reported an error on launch */
} vsa_status;

/* ----- element types ------------------------------------------------------ */
typedef enum vsa_dtype {
  VSA_F32 = 0,       /* IEEE float32 */
  VSA_BF16 = 1,      /* bfloat16 */
  VSA_FP8_E4M3 = 2,  /* OCP FP8 E4M3 ("fn": bias 7, max 448, no inf) codes + fp32 tile scales */
  /* As VSA_FP8_E4M3, with the V codes in the P.V operand layout written by
   * vsa_quant_fp8_tiles_v (attention only; Q and K codes as before). */
  VSA_FP8_E4M3_VOP = 3,
  /* As VSA_BF16, with V in the bf16 P.V operand layout written by
   * vsa_tile_permute_v (attention forwards only; Q and K tiled as before). */
  VSA_BF16_VOP = 4
} vsa_dtype;

/* ----- token layouts ------------------------------------------------------ */
typedef enum vsa_layout_kind {
  /* 3D tiles of tile_t x tile_h x tile_w tokens. Each axis is padded at its
   * high end to a multiple of the tile extent; tiles are numbered row-major
   * over tile coordinates, tokens row-major (t, h, w) inside a tile. */
  VSA_TILE3D = 0,
  /* Skiparse-2D residue groups: token (t, h, w) belongs to group
   * g = (h mod stride_h) * stride_w + (w mod stride_w). Groups are stored one
   * after another, each row-major over (t, h / stride_h, w / stride_w), and
   * cut into chunks of tile_t * tile_h * tile_w tokens; a group's last chunk
   * is padded. Requires H % stride_h == 0 and W % stride_w == 0. */
  VSA_SKIPARSE2D = 1
} vsa_layout_kind;

typedef struct vsa_layout {
  int32_t batch;      /* B >= 1 */
  int32_t heads;      /* attention heads >= 1 */
  int32_t head_dim;   /* d */
  int32_t T, H, W;    /* latent grid, each >= 1 */
  int32_t kind;       /* vsa_layout_kind */
  int32_t tile_t, tile_h, tile_w;  /* tile extents (>= 1); tile tokens = product */
  int32_t stride_h, stride_w;      /* Skiparse strides (>= 1); ignored for VSA_TILE3D */
} vsa_layout;

typedef struct vsa_layout_info {
  int64_t n_tokens;        /* T * H * W */
  int64_t n_padded;        /* n_tiles * tile_tokens: rows of a tiled tensor per (b, head) */
  int32_t n_tiles;         /* tiles per (b, head) */
  int32_t tile_tokens;     /* tile_t * tile_h * tile_w */
  int32_t n_groups;        /* Skiparse residue groups (1 for VSA_TILE3D) */
  int32_t tiles_per_group; /* tiles of one group (n_tiles for VSA_TILE3D) */
  int32_t group_len;       /* real tokens of one group (n_tokens for VSA_TILE3D) */
  int32_t tiles_t, tiles_h, tiles_w; /* 3D tile grid (VSA_TILE3D; zeros otherwise) */
} vsa_layout_info;

/* Derives the padded sizes of a layout (host only, no GPU work).
 * Returns VSA_ERR_INVALID for non-positive sizes or a Skiparse grid that the
 * strides do not divide. */
vsa_status vsa_layout_query(const vsa_layout* layout, vsa_layout_info* info);

/* ----- S1 / S7: tile permutation -------------------------------------------
 * FPSAttention, Approach (shared 3D tile granularity); FVAttn summary
 * (video-aware block organisation); OSP-Next card, Model Summary (Skiparse
 * groups along H and W).
 *   inverse == 0: src natural [B, T*H*W, heads, d] -> dst tiled [B, heads, n_padded, d];
 *                 pad rows of dst are written as zeros.
 *   inverse != 0: src tiled [B, heads, n_padded, d] -> dst natural [B, T*H*W, heads, d];
 *                 pad rows of src are ignored.
 * dtype: VSA_F32 or VSA_BF16 (d * element size must be a multiple of 16 bytes).
 * The result is a pure data movement: bit-exact. src and dst must not overlap. */
vsa_status vsa_tile_permute(const vsa_layout* layout, int32_t dtype, const void* src, void* dst,
                            int32_t inverse, void* stream);

/* vsa_tile_permute_v: the tile permutation of a bf16 V (FVAttn summary:
 * video-aware block organisation), stored in the order the bf16 P.V product
 * of the forward consumes it, so the kernel stages V with whole 16-byte
 * copies. src bf16 natural [B, T*H*W, heads, d] -> dst bf16 [B, heads,
 * n_padded, d]: tile j of (b, head) occupies elements [64*d*j, 64*d*(j+1))
 * of its slice as two 32-token blocks kb = 0, 1 of 32*d elements; element
 * 32*c + p of block kb holds channel c of the tile's token
 * 32*kb + 16*A + 8*(i / 4) + 4*h + i % 4, where p = 16*A + 8*h + i
 * (A, h in 0..1; i in 0..7). Pad tokens are written as zeros. A pure data
 * movement (bit-exact). Needs tile_tokens 64 and head_dim <= 256 and a
 * multiple of 8 (VSA_ERR_UNSUPPORTED otherwise); 16-byte aligned pointers;
 * src and dst must not overlap. Pass the result as v with dtype VSA_BF16_VOP. */
vsa_status vsa_tile_permute_v(const vsa_layout* layout, const void* src, void* dst, void* stream);

/* ----- S2: fixed block masks -------------------------------------------------
 * FPSAttention, Approach and window ablation (sliding tile window);
 * OSP-Next card, Model Summary (Skiparse-2D; full-attention layers).
 * Writes one head-invariant list per query tile:
 *   kv_idx int32 [n_tiles, max_kv]: ascending key-tile indices (slots past the
 *                                   count are left untouched),
 *   kv_cnt int32 [n_tiles].
 * VSA_TILE3D: key tile kept iff |delta| <= (rt, rh, rw) per axis in tile
 *   coordinates, clipped at the grid edge.
 * VSA_SKIPARSE2D: every tile of the query tile's residue group (radii unused).
 * Any negative radius: dense, every tile listed.
 * VSA_ERR_INVALID if max_kv is smaller than the longest list. */
vsa_status vsa_build_mask_window(const vsa_layout* layout, int32_t rt, int32_t rh, int32_t rw,
                                 int32_t max_kv, int32_t* kv_idx, int32_t* kv_cnt, void* stream);

/* ----- big tiles: grouped windows ---------------------------------------------
 * FPSAttention (Approach, and its ablation table): sparsity and quantisation
 * share one tile granularity, changed across denoising steps; larger,
 * hardware-friendly (6,8,8) tiles and asymmetric windows such as (6,6,1).
 * A big tile is a group of gt x gh x gw consecutive tiles of a VSA_TILE3D
 * layout (e.g. (6,1,1) groups of (1,8,8) tiles = (6,8,8) tiles, the last
 * group along an axis possibly shorter), so the attention kernels keep their
 * 64-token tiles. A window extent e (per axis, >= 1) counts groups: around
 * the query tile's group X it covers groups X - (e-1)/2 .. X - (e-1)/2 + e - 1
 * (integer division; the extra group of an even extent on the high side),
 * clipped at the grid edge without shifting. Each query tile lists every
 * tile of every covered group, ascending.
 *   kv_idx int32 [n_tiles, max_kv], kv_cnt int32 [n_tiles] (head-invariant,
 *   list_mode 0 for the attention call).
 * VSA_ERR_INVALID if max_kv is smaller than the longest list, a group size or
 * an extent is < 1; VSA_ERR_UNSUPPORTED for VSA_SKIPARSE2D layouts. */
vsa_status vsa_build_mask_window_grouped(const vsa_layout* layout, int32_t gt, int32_t gh,
                                         int32_t gw, int32_t et, int32_t eh, int32_t ew,
                                         int32_t max_kv, int32_t* kv_idx, int32_t* kv_cnt,
                                         void* stream);

/* ----- S3 / S4: adaptive routing ---------------------------------------------
 * VSA page, Research Type row (coarse selection of key blocks per query
 * block); FVAttn summary (Top-p routing with a Top-k safety floor, per head).
 *   q_tiled, k_tiled: bf16 [B, heads, n_padded, d] (output of vsa_tile_permute).
 * Steps, per (b, head):
 *   pooled tile means over real (non-pad) tokens, in fp32;
 *   s_ij = coarse_scale * <qbar_i, kbar_j> (fp32, the products accumulated
 *   in a fixed channel order, the same on every call);
 *   top_p <= 0: keep the top_k highest-scoring key tiles (ties: lower index);
 *   top_p  > 0: p_ij = softmax_j(s_ij); keep the shortest prefix of the
 *               descending order whose mass reaches top_p, then at least
 *               k_floor tiles (capped at n_tiles); top_k is unused. The mass
 *               of a prefix is an fp32 sum in a fixed order, so where the
 *               exact mass at the cut lies within rounding of top_p the count
 *               may differ by one from an exact evaluation.
 * Scores and selection run in one pass: no n_tiles x n_tiles buffer is
 * formed unless `scores` is requested.
 * Outputs: kv_idx int32 [B, heads, n_tiles, max_kv] ascending, kv_cnt int32
 *   [B, heads, n_tiles]; scores (optional, may be NULL) float [B, heads,
 *   n_tiles, n_tiles] holding s_ij.
 * workspace: device memory of at least vsa_build_mask_topk_workspace() bytes
 *   (the pooled means of Q and K), 16-byte aligned.
 * Limits: n_tiles <= 4096, head_dim <= 256 and a multiple of 8.
 * Deterministic: repeated calls give identical lists.
 * VSA_ERR_INVALID if max_kv < the largest possible count (top_k, or n_tiles
 * for top-p). */
vsa_status vsa_build_mask_topk(const vsa_layout* layout, const void* q_tiled, const void* k_tiled,
                               float coarse_scale, int32_t top_k, float top_p, int32_t k_floor,
                               int32_t max_kv, int32_t* kv_idx, int32_t* kv_cnt, float* scores,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes vsa_build_mask_topk needs for this layout: 2 * B * heads *
 * n_tiles * head_dim * 4 (0 on a bad layout). */
size_t vsa_build_mask_topk_workspace(const vsa_layout* layout);

/* S1 with S3 folded in: FVAttn summary (video-aware block organisation: the
 * pooling is a by-product of the regrouping pass); VSA page, Research Type row
 * (the coarse stage works on pooled blocks).
 *   src bf16 [B, T*H*W, heads, d] natural order -> dst bf16 [B, heads,
 *   n_padded, d] tiled (bit-identical to vsa_tile_permute, pads zero) and
 *   pooled float [B, heads, n_tiles, d]: each tile's mean over its real
 *   tokens, the same fp32 values, bit for bit, as the pooling step inside
 *   vsa_build_mask_topk (0 for a tile without real tokens).
 * dst may be NULL: the means only (for a Q read by the natural-order
 * forward, which needs no tiled copy).
 * One pass over the tensor instead of the permute's pass plus the pool's.
 * src, dst and pooled 16-byte aligned; buffers must not overlap.
 * VSA_ERR_UNSUPPORTED unless head_dim <= 256 and a multiple of 8. */
vsa_status vsa_tile_permute_pool(const vsa_layout* layout, const void* src, void* dst,
                                 float* pooled, void* stream);

/* S4 from pooled means: vsa_build_mask_topk's scoring and selection (same
 * rules, limits and outputs) on q_pooled and k_pooled, float [B, heads,
 * n_tiles, d] as written by vsa_tile_permute_pool (16-byte aligned). Given
 * the means that vsa_build_mask_topk would pool from the same Q and K, the
 * lists and scores are bit-identical to its. Needs no workspace: workspace
 * and workspace_bytes are ignored (NULL and 0 are fine). */
vsa_status vsa_build_mask_topk_pooled(const vsa_layout* layout, const float* q_pooled,
                                      const float* k_pooled, float coarse_scale, int32_t top_k,
                                      float top_p, int32_t k_floor, int32_t max_kv,
                                      int32_t* kv_idx, int32_t* kv_cnt, float* scores,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* ----- S5: per-tile fp8 quantiser ---------------------------------------------
 * FPSAttention, Approach (FP8 on the same 3D tiles as the sparsity).
 *   x_tiled bf16 [B, heads, n_padded, d] -> codes uint8 [B, heads, n_padded, d]
 *   (OCP E4M3) and scales float [B, heads, n_tiles].
 * Per (b, head, tile): a = absmax over real tokens and all d channels;
 *   scale = fl32(a / 448); code = RNE_e4m3(fl32(x * fl32(448 / a))), saturating;
 *   a == 0 gives scale 0 and zero codes; pad rows get code 0.
 * Bit-exact: the operation sequence is fixed in fp32. */
vsa_status vsa_quant_fp8_tiles(const vsa_layout* layout, const void* x_tiled, uint8_t* codes,
                               float* scales, void* stream);

/* Same quantisation (bit-identical codes and scales) with the codes of each
 * tile stored channel-major in the order the fp8 P.V product consumes V
 * (FPSAttention, Approach: P.V in FP8): tile j of (b, head) occupies bytes
 * [64*128*j, 64*128*(j+1)) of its [n_padded, d] slice; byte 64*c + p holds
 * channel c of the tile's token t = 32*A + 8*B + 4*h + r, where position
 * p = 32*h + 16*A + 4*B + r (h, A in 0..1; B, r in 0..3). Pad tokens have
 * code 0. Needs tile_tokens 64 and head_dim 128 (VSA_ERR_UNSUPPORTED
 * otherwise); codes must be 16-byte aligned. Pass the result as v with
 * dtype VSA_FP8_E4M3_VOP. */
vsa_status vsa_quant_fp8_tiles_v(const vsa_layout* layout, const void* x_tiled, uint8_t* codes,
                                 float* scales, void* stream);

/* vsa_quant_fp8_tiles_grouped: as vsa_quant_fp8_tiles (v_operand 0) or
 * vsa_quant_fp8_tiles_v (v_operand 1), with one scale per big tile: a is the
 * absmax over the real tokens of all gt x gh x gw tiles of the group (see
 * vsa_build_mask_window_grouped), and the group's scale fl32(a / 448) is
 * written for each of its tiles, so the attention call takes the result
 * unchanged (FPSAttention, Approach: FP8 on the same tiles as the sparsity).
 * VSA_TILE3D layouts only; VSA_ERR_INVALID for group sizes < 1. */
vsa_status vsa_quant_fp8_tiles_grouped(const vsa_layout* layout, int32_t gt, int32_t gh, int32_t gw,
                                       const void* x_tiled, uint8_t* codes, float* scales,
                                       int32_t v_operand, void* stream);

/* vsa_quant_fp8_tiles_nat: S1 and S5 (and S3) in one pass (FVAttn summary:
 * video-aware block organisation; FPSAttention, Approach: FP8 on the shared
 * tiles). x_nat bf16 [B, T*H*W, heads, d] in the natural order -> codes and
 * scales bit-identical to vsa_tile_permute followed by vsa_quant_fp8_tiles
 * (v_operand 0) or vsa_quant_fp8_tiles_v (v_operand 1); no tiled bf16 copy
 * is written. pooled (may be NULL) float [B, heads, n_tiles, d]: also the
 * tile means, bit-identical to vsa_tile_permute_pool's, for routing.
 * Needs head_dim <= 256 and a multiple of 8 and tile_tokens * head_dim <=
 * 16,384 (the P.V operand layout: 64-token tiles and head_dim 128),
 * VSA_ERR_UNSUPPORTED otherwise; x_nat and pooled 16-byte aligned, codes 8
 * (16 for the operand layout). */
vsa_status vsa_quant_fp8_tiles_nat(const vsa_layout* layout, const void* x_nat, uint8_t* codes,
                                   float* scales, float* pooled, int32_t v_operand, void* stream);

/* ----- S6: block-sparse attention forward --------------------------------------
 * The flash-style, FlashAttention-compatible sparse attention every page
 * builds on (OSP-Next wiki TL;DR; FPSAttention, Approach; VSA, Research
 * Type row; FVAttn summary). For every real query token i of query tile Q:
 *   O_i = sum_{j in A(i)} exp(sigma q_i.k_j) v_j / sum_{j in A(i)} exp(sigma q_i.k_j)
 * with A(i) the real key tokens of the key tiles listed for Q.
 *   q, k, v: tiled [B, heads, n_padded, d]
 *     dtype VSA_F32: float inputs (rounded to bf16 for the products), float out;
 *     dtype VSA_BF16: bf16 in, bf16 out;
 *     dtype VSA_FP8_E4M3: uint8 codes in with q_scale / k_scale / v_scale
 *       float [B, heads, n_tiles] from vsa_quant_fp8_tiles; bf16 out;
 *     dtype VSA_FP8_E4M3_VOP: the same, with v from vsa_quant_fp8_tiles_v
 *       (no byte transposition of V inside the kernel; identical output);
 *     dtype VSA_BF16_VOP: as VSA_BF16, with v from vsa_tile_permute_v
 *       (64-token tiles; output identical to VSA_BF16's).
 *   kv_idx / kv_cnt: lists as written by vsa_build_mask_window (list_mode 0:
 *     one table [n_tiles, max_kv] shared by every batch and head) or by
 *     vsa_build_mask_topk (list_mode 1: [B, heads, n_tiles, max_kv]).
 *     list_mode 2 takes a list_mode 0 table but walks each query tile's list
 *     on its own instead of four neighbouring tiles' union (faster where
 *     neighbouring query tiles share few key tiles, e.g. narrow big-tile
 *     windows); the result is the same.
 *     Both NULL: dense attention (every tile). Indices must lie in
 *     [0, n_tiles) and counts in [0, max_kv]; the kernel does not re-check them.
 *   work_order (optional, may be NULL; list_mode 1 only, VSA_ERR_INVALID
 *     otherwise): int32 [B * heads * n_tiles] from vsa_build_work_order, the
 *     order in which the (b, head, query tile) walks are dealt to the
 *     workgroups. It changes only the schedule: the output is bit-identical
 *     with or without it. Entries are clamped into range; an array that is
 *     not a permutation leaves some tiles unwritten but cannot fault.
 *   out: [B, heads, n_padded, d]; pad query rows and rows with an empty list
 *     are written as 0.
 *   lse (optional, may be NULL): float [B, heads, n_padded], natural-log
 *     sum_{j in A(i)} exp(sigma q_i.k_j); -inf for pad rows and empty lists.
 * Supported: tile_tokens in {32, 64}; head_dim in {64, 128}; the fp8 dtypes
 * need tile_tokens 64 and head_dim 128; one (batch, head) slice of q, k or v
 * (n_padded * d elements) must stay below 2 GiB, as the kernels address it
 * with 32-bit offsets (VSA_ERR_UNSUPPORTED otherwise; the same holds for the
 * natural-order forward and the backward). */
vsa_status vsa_block_sparse_attn_fwd(const vsa_layout* layout, int32_t dtype, const void* q,
                                     const void* k, const void* v, const float* q_scale,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* kv_idx, const int32_t* kv_cnt, int32_t max_kv,
                                     int32_t list_mode, const int32_t* work_order,
                                     float softmax_scale, void* out, float* lse, void* stream);

/* vsa_build_work_order: S6's heavy-first dealing of routed work (FVAttn
 * summary, Summary and Abstract: Top-p routing makes the work per head, and
 * per query tile, uneven). From the counts kv_cnt int32 [B, heads, n_tiles]
 * of per-head lists (list_mode 1) writes order int32 [B * heads * n_tiles],
 * a permutation of the items b * heads * n_tiles + head * n_tiles + t:
 *   (b, head) slices by their total max(cnt, 0) (each count clamped to
 *   n_tiles), descending, equal totals in index order; within a slice, query
 *   tiles by count, descending, equal counts in index order.
 * Deterministic (integer keys and ranks). Needs n_tiles + B * heads <=
 * 16,384 (VSA_ERR_UNSUPPORTED otherwise); kv_cnt and order 4-byte aligned
 * and not overlapping. */
vsa_status vsa_build_work_order(const vsa_layout* layout, const int32_t* kv_cnt, int32_t* order,
                                void* stream);

/* vsa_block_sparse_attn_fwd_nat: vsa_block_sparse_attn_fwd with the tile
 * permute of Q and the inverse permute of O fused into the kernel (one
 * full-tensor pass each saved; FVAttn summary: video-aware block
 * organisation of the tokens). q and out are in the natural order
 * [B, T*H*W, heads, d]; k and v stay tiled [B, heads, n_padded, d] (from
 * vsa_tile_permute); lse, if given, is in the tiled order as for the
 * forward. Every real token of out is written; the result equals the
 * forward's followed by vsa_tile_permute(inverse). dtype VSA_F32, VSA_BF16
 * or VSA_BF16_VOP (VSA_ERR_UNSUPPORTED otherwise, and when one batch of q exceeds
 * 2 GiB); lists, list_mode, work_order and scale as for
 * vsa_block_sparse_attn_fwd. */
vsa_status vsa_block_sparse_attn_fwd_nat(const vsa_layout* layout, int32_t dtype, const void* q,
                                         const void* k, const void* v, const int32_t* kv_idx,
                                         const int32_t* kv_cnt, int32_t max_kv, int32_t list_mode,
                                         const int32_t* work_order, float softmax_scale, void* out,
                                         float* lse, void* stream);

/* vsa_block_sparse_attn_fwd_fp8_nat: the fp8 forward (dtype VSA_FP8_E4M3 or
 * VSA_FP8_E4M3_VOP; q, k, v tiled codes with their scales, lists, list_mode,
 * work_order and scale as for vsa_block_sparse_attn_fwd) with the inverse tile permute
 * of O folded into the kernel's last store: out is bf16 in the natural order
 * [B, T*H*W, heads, d], every real token written (FVAttn summary:
 * video-aware block organisation). lse, if given, is tiled as for the
 * forward. The result equals vsa_block_sparse_attn_fwd followed by
 * vsa_tile_permute(inverse), bit for bit. Needs 64-token tiles and head_dim
 * 128 (VSA_ERR_UNSUPPORTED otherwise). */
vsa_status vsa_block_sparse_attn_fwd_fp8_nat(const vsa_layout* layout, int32_t dtype, const void* q,
                                             const void* k, const void* v, const float* q_scale,
                                             const float* k_scale, const float* v_scale,
                                             const int32_t* kv_idx, const int32_t* kv_cnt,
                                             int32_t max_kv, int32_t list_mode,
                                             const int32_t* work_order, float softmax_scale,
                                             void* out, float* lse, void* stream);

/* ----- S6 backward: gradients of the block-sparse attention -------------------
 * The pages train through this attention: VSA ("Faster Video Diffusion with
 * Trainable Sparse Attention", Research Type and Experiment Setup rows) is a
 * trainable sparse attention used to pretrain and fine-tune video DiTs, and
 * FPSAttention (Approach) trains jointly with FP8 and tile sparsity. The
 * gradients are the chain rule of the forward's definition: for real query
 * token i with key set A(i), P_ij = exp(sigma q_i.k_j - lse_i) and
 * D_i = dO_i . O_i,
 *   dV_j = sum_i P_ij dO_i,   dS_ij = P_ij (dO_i.v_j - D_i),
 *   dQ_i = sigma sum_j dS_ij k_j,   dK_j = sigma sum_i dS_ij q_i.
 *
 * vsa_build_transposed_lists: for every key tile j, the ascending query
 * tiles whose list holds j (the walk order of the dK/dV kernel).
 *   kv_idx / kv_cnt: forward lists as for vsa_block_sparse_attn_fwd
 *     (list_mode 0: [n_tiles, max_kv]; 1: [B, heads, n_tiles, max_kv]); each
 *     list must be strictly ascending (as the mask builders write them).
 *   q_idx: int32 [LH, n_tiles, n_tiles] and q_cnt: int32 [LH, n_tiles],
 *     LH = 1 (list_mode 0) or B * heads (list_mode 1). Row j of q_idx holds
 *     q_cnt[j] query tiles; the rest of the row is left unwritten.
 * Deterministic; builds once per set of lists and may be cached with them. */
vsa_status vsa_build_transposed_lists(const vsa_layout* layout, const int32_t* kv_idx,
                                      const int32_t* kv_cnt, int32_t max_kv, int32_t list_mode,
                                      int32_t* q_idx, int32_t* q_cnt, void* stream);

/* Bytes of device workspace vsa_block_sparse_attn_bwd needs: 8 bytes per
 * padded row of every (batch, head); 0 for an invalid layout. */
size_t vsa_block_sparse_attn_bwd_workspace(const vsa_layout* layout);

/* vsa_block_sparse_attn_bwd: dq, dk, dv of the forward call with the same
 * layout, dtype, q, k, v, lists and softmax_scale.
 *   dtype: VSA_BF16 (bf16 tensors and gradients) or VSA_F32 (float tensors,
 *     rounded to bf16 for the products; float gradients).
 *   out, lse: the forward's output and its (non-NULL) lse.
 *   dout: upstream gradient of out, tiled [B, heads, n_padded, d]; its pad
 *     rows are ignored.
 *   kv_idx / kv_cnt / max_kv: the forward lists; q_idx / q_cnt: their
 *     transposition from vsa_build_transposed_lists with the same list_mode.
 *     All four NULL: dense attention.
 *   dq, dk, dv: [B, heads, n_padded, d], fully written: pad rows get 0. They
 *     must not alias the inputs.
 *   workspace: device memory of at least vsa_block_sparse_attn_bwd_workspace()
 *     bytes (VSA_ERR_WORKSPACE otherwise), 8-byte aligned.
 * Supported: tile_tokens in {32, 64}; head_dim in {64, 128}. No atomics:
 * repeated calls give bit-identical results. */
vsa_status vsa_block_sparse_attn_bwd(const vsa_layout* layout, int32_t dtype, const void* q,
                                     const void* k, const void* v, const void* out,
                                     const void* dout, const float* lse, const int32_t* kv_idx,
                                     const int32_t* kv_cnt, int32_t max_kv, const int32_t* q_idx,
                                     const int32_t* q_cnt, int32_t list_mode, float softmax_scale,
                                     void* dq, void* dk, void* dv, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* vsa_block_sparse_attn_bwd_noalloc: vsa_block_sparse_attn_bwd (same
 * arguments, checks and results, bit for bit) without a workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight training or serving loops, harnesses that forbid allocation. The row
 * statistics live in a 32 MiB scratch array built into the library, one copy
 * on every GPU it runs on, held until the process ends; the call allocates
 * nothing. Limit: B * heads * n_padded <= 4,194,304 rows (8 bytes each; the
 * 768p Skiparse layer with 40 heads needs 3,225,600), VSA_ERR_UNSUPPORTED
 * beyond it. Calls on one GPU share that scratch: calls that overlap in time
 * on one GPU (different streams, or threads) race and must not be issued. */
vsa_status vsa_block_sparse_attn_bwd_noalloc(const vsa_layout* layout, int32_t dtype, const void* q,
                                             const void* k, const void* v, const void* out,
                                             const void* dout, const float* lse,
                                             const int32_t* kv_idx, const int32_t* kv_cnt,
                                             int32_t max_kv, const int32_t* q_idx,
                                             const int32_t* q_cnt, int32_t list_mode,
                                             float softmax_scale, void* dq, void* dk, void* dv,
                                             void* stream);

/* ----- diagnostics --------------------------------------------------------- */
const char* vsa_status_string(int32_t status);
/* Message for the last failing call on this thread ("" if none). */
const char* vsa_last_error(void);
/* Library version, "major.minor.patch". */
const char* vsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H_ */

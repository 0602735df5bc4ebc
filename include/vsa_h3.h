/*
 * vsa_h3.h -- C ABI of the VSA-H3 attention forward for AMD Instinct MI355X
 * (gfx950).
 *
 * The operation (FastH3 4-step Preview (VSA, data-free), section "Video
 * Sparse Attention is not optional here"): packed tokens [text | cond |
 * audio | video] are cut into 64-token tiles -- segment-pure prefix tiles
 * and (4,4,4) tiles over the post-patchify video grid -- derived from token
 * tags and positions.  Per head, mean-pooled q and k give fp32 tile scores;
 * every video query tile keeps the top-k video key tiles,
 *     topk = max(1, min(ceil((1 - sparsity) * n_video_tiles), n_video_tiles)),
 * plus every prefix key tile; prefix query tiles attend to all tiles.  The
 * fine branch is block-sparse softmax attention over the kept tiles (FastH3
 * NVFP4 on RTX PRO 6000, "Block-sparse FP4 attention for VSA tiles").  A
 * compression branch softmax(scores) @ pool(v) is broadcast over each query
 * tile's rows, multiplied by a per-token gate with no activation, and added.
 * The output returns to packed order ("Model integration" on the same page).
 *
 * The OmniRef page ("Device profiles") also runs VSA with 128-token tiles
 * and a reference keep ratio; both are options here: a video tile may be any
 * box of 128 grid cells (prefix tiles then hold 128 tokens), and with keep
 * ratio r < 1 (vsa_h3_plan_set_ref_keep) each video query tile visits only
 * its best-scoring reference (cond) key tiles among the prefix tiles.
 *
 * Conventions shared by every entry point
 *   - Every call returns a vsa_status; on failure vsa_h3_last_error() holds a
 *     message (thread-local, valid until the next call on the same thread).
 *     There is no fallback route: an unsupported request is an error.
 *   - Device buffers are caller-owned.  The library never allocates or frees
 *     device memory; intermediates live in a caller-provided workspace whose
 *     size vsa_h3_plan_info() reports.
 *   - Device work is only enqueued on `stream` (a hipStream_t passed as
 *     void*; NULL is the null stream).  Calls do not synchronize, except that
 *     vsa_h3_plan_upload copies from pageable host memory.
 *   - The forwards (vsa_h3_forward, vsa_h3_forward_qk_prep) enqueue kernel
 *     launches only: no allocation, no memset, no copy, no host wait.  After
 *     vsa_h3_plan_upload has filled a workspace they may be captured in a
 *     HIP graph on `stream` and replayed; every workspace region other than
 *     the uploaded tables is written before it is read within one forward.
 *   - Tensors are contiguous, sequence-major [L][heads][head_dim] (batch 1).
 *   - Indices are int32 on the device (L < 2^31); byte offsets are 64-bit.
 */
#ifndef VSA_H3_H
#define VSA_H3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VSA_OK = 0,
  VSA_E_ARG = -1,          /* bad argument: NULL pointer, size, sparsity outside [0,1] */
  VSA_E_LAYOUT = -2,       /* token tags: unknown tag, or a video token before a prefix token */
  VSA_E_POSITIONS = -3,    /* video positions outside the grid, duplicated, or not covering it */
  VSA_E_UNSUPPORTED = -4,  /* head_dim, tile shape or size outside what the kernels implement */
  VSA_E_WORKSPACE = -5,    /* workspace NULL, misaligned or smaller than vsa_h3_info.workspace_bytes */
  VSA_E_HIP = -6           /* a HIP runtime call or kernel launch failed */
} vsa_status;

typedef enum { VSA_BF16 = 0, VSA_F32 = 1 } vsa_dtype;

/* Segment tags of the packed stream (int64 on the wire). */
enum { VSA_TAG_TEXT = 0, VSA_TAG_COND = 1, VSA_TAG_AUDIO = 2, VSA_TAG_VIDEO = 3 };

typedef struct { int32_t t, h, w; } vsa_dims3;

typedef struct vsa_h3_plan vsa_h3_plan;   /* opaque; host memory owned by the library */

typedef struct {
  int64_t L;                 /* tokens */
  int64_t num_prefix_tiles;  /* P: prefix tiles, ids 0..P-1 */
  int64_t num_video_tiles;   /* NV: video tiles, ids P..P+NV-1 */
  int64_t num_tiles;         /* Nt = P + NV */
  int64_t topk;              /* video key tiles kept per video query tile (0 if NV == 0) */
  int32_t heads, head_dim;
  uint64_t workspace_bytes;  /* bytes the workspace must hold */
  int32_t chunk_tiles;       /* key tiles per fine-branch key chunk */
  int32_t num_chunks;        /* key chunks, ceil(num_tiles / chunk_tiles); 0 if num_tiles == 0 */
  int64_t num_ref_tiles;     /* prefix tiles of tag cond (reference tiles) */
  int64_t topk_ref;          /* reference tiles kept per video query tile by the selection;
                                0 when the keep ratio is 1 (every reference tile visited) */
  double ref_keep;           /* reference keep ratio, 1 by default */
  int32_t tile_tokens;       /* tokens per tile: 64 or 128 */
  int32_t num_blocks;        /* 64-slot blocks, num_tiles * tile_tokens / 64 */
} vsa_h3_info;

/* Byte offsets of the intermediates inside the workspace (each 256-aligned).
 * They are documented so that tests and tools can read intermediates back;
 * their contents are only meaningful after a forward on the same stream.
 * Token-level regions are laid out in 64-slot blocks: Nb = num_blocks blocks,
 * one per 64-token tile, or two per 128-token tile (slots 0-63, then 64-127). */
typedef struct {
  uint64_t perm;    /* int32 [Nb][64]: packed row of each slot, -1 for pad slots */
  uint64_t valid;   /* int32 [Nb]: valid tokens per block */
  uint64_t kt;      /* bf16 [H][Nb][2][D/32][32][32]: keys in tile order, pad rows zero; per
                       block, each half of 32 slots (0-31, 32-63) is stored group by group,
                       a group holding 32 channels (64 bytes) of its 32 key rows */
  uint64_t vt;      /* bf16 [H][Nb][2][D][32]: values in tile order, transposed, in two halves
                       of 32 slots (0-31, 32-63) per block, pad columns zero; inside each
                       16-slot group the columns hold slots 0-3, 8-11, 4-7, 12-15 */
  uint64_t qp;      /* fp32 [H][Nt][D]: pooled (mean) q per tile */
  uint64_t kp;      /* fp32 [H][Nt][D]: pooled k */
  uint64_t vp;      /* fp32 [H][Nt][D]: pooled v */
  uint64_t scores;  /* fp32 [H][Nt][Ns]: tile scores, Ns = Nt rounded up to 4; after the
                       forward each row holds softmax(scores / sqrt(D)) instead */
  uint64_t coarse;  /* fp32 [H][Nt][D]: compression output per query tile */
  uint64_t sel;     /* int32 [H][NV][topk_ref + topk]: selected key tiles, ascending (the
                       selected reference tiles, then the selected video tiles) */
  uint64_t total;   /* == vsa_h3_info.workspace_bytes */
  int64_t scores_row_stride;  /* Ns */
  uint64_t chunk_offsets;  /* int32 [H][NV][num_chunks + 1] (only if num_chunks > 1): entry c
                              counts the listed tiles of the row with id < c * chunk_tiles (the
                              selected video tiles, or with topk_ref > 0 the visit list) */
  uint64_t state;   /* fp32 fine-branch state between key chunks (only if num_chunks > 1);
                       internal layout */
  uint64_t qt;      /* bf16 [H][Nb][64][D]: q after QK-norm + RoPE, tile order, pad rows zero
                       (only with vsa_h3_plan_set_qk_prep) */
  uint64_t kt8;     /* uint8 [H][Nb][2][D/64][32][64]: keys as OCP E4M3 codes, tile order, pad
                       rows zero, in the half and group order of kt (a group holds 64 codes)
                       (only with vsa_h3_plan_set_qk_fp8) */
  uint64_t kscale;  /* fp32 [H][Nb][64]: per-key dequantisation scale amax/448, pad slots zero
                       (only with vsa_h3_plan_set_qk_fp8) */
  uint64_t kind;    /* int32 [Nt]: 0 prefix tile visited by every query, 1 reference (cond)
                       tile, 2 video tile */
  uint64_t visit;   /* int32 [H][NV][V] (only if topk_ref > 0): every key tile a video query
                       tile visits, ascending: the non-reference prefix tiles, the selected
                       reference tiles and the selected video tiles,
                       V = (num_prefix_tiles - num_ref_tiles) + topk_ref + topk */
  uint64_t order;   /* int32 [H][num_chunks][Nt] (only if num_chunks > 1): the query tiles of
                       each head in the order the fine branch dispatches them for each key
                       chunk, most visits in the chunk first (ties in no fixed order) */
  uint64_t kt_lo;   /* bf16, layout of kt (only for fp32 I/O, without FP8 keys): the low part
                       bf16(x - bf16(x)) of every key element */
  uint64_t vt_lo;   /* bf16, layout of vt (only for fp32 I/O): low parts of the values */
  uint64_t qt_lo;   /* bf16, layout of qt (only for fp32 I/O with QK-norm + RoPE): low parts
                       of the normalised, rotated queries */
} vsa_h3_ws_layout;

/* Top-k rule of VSA-H3 evaluated in IEEE double as written; 0 when
 * num_video_tiles <= 0; -1 if sparsity is outside [0, 1] or NaN. */
int64_t vsa_h3_topk(int64_t num_video_tiles, double sparsity);

/* Build the tile geometry (host only; touches no GPU).
 *   token_tags    host int64 [L], values VSA_TAG_*; every non-video token must
 *                 precede every video token.  Each maximal run of one prefix
 *                 tag is a segment, cut into 64-token tiles in packed order
 *                 (the last tile of a segment may be partial).
 *   position_ids  host int64 [L][3] (t, y, x), zero-based; read for video
 *                 tokens only, which must cover grid exactly once.
 *   grid          post-patchify video grid (T, H, W); T*H*W must equal the
 *                 number of video tokens.
 *   tile          (tt, th, tw) >= 1 with tt*th*tw = 64 (the pages' (4,4,4)) or
 *                 128 (the OmniRef page's 128-token tiles; the pages do not
 *                 give the box, (4,8,4) divides the 480p and 768p grids).
 *                 Prefix tiles hold tt*th*tw tokens.
 *   heads >= 1; head_dim 64 or 128; sparsity in [0, 1].
 * Video tile of (t,y,x): P + ((t/tt)*ceil(H/th) + y/th)*ceil(W/tw) + x/tw;
 * slot order inside a tile is the (t,y,x) raster of its valid cells.  Edge
 * tiles may be partial.  VSA_E_UNSUPPORTED for another tile volume.  On
 * success *plan_out owns host memory until vsa_h3_plan_destroy. */
vsa_status vsa_h3_plan_create(const int64_t* token_tags, const int64_t* position_ids,
                              int64_t L, vsa_dims3 grid, vsa_dims3 tile, int32_t heads,
                              int32_t head_dim, double sparsity, vsa_h3_plan** plan_out);

vsa_status vsa_h3_plan_info(const vsa_h3_plan* plan, vsa_h3_info* out);

/* Key chunking of the fine branch (a schedule choice; the result does not
 * depend on it beyond fp32 rounding of the running softmax state).  Each
 * query tile visits its key tiles in ascending id order; the visit list is
 * cut at multiples of chunk_tiles and the chunks run as consecutive kernel
 * launches, so that all query tiles of a head sweep one chunk of its K/V
 * together while it stays cached (L2 and Infinity Cache).  The running max, running
 * sum and unnormalised output of every query row pass between launches
 * through the workspace, in fp32.
 *   chunk_tiles  0 picks the default (chunks of at most 10 MiB of K+V per
 *                head with 64-token tiles, 32 MiB with 128-token tiles,
 *                balanced; with FP8 q/k the keys count one byte per
 *                element); otherwise the chunk length in key tiles.
 * The workspace size changes: call before sizing and uploading a workspace.
 * VSA_E_ARG if chunk_tiles < 0 or if it gives more than 63 chunks. */
vsa_status vsa_h3_plan_set_chunk_tiles(vsa_h3_plan* plan, int32_t chunk_tiles);
vsa_status vsa_h3_plan_layout(const vsa_h3_plan* plan, vsa_h3_ws_layout* out);

/* I/O dtype the workspace is laid out for (VSA_BF16 by default).  A forward
 * with io_dtype VSA_F32 needs a plan set to VSA_F32: its workspace also holds
 * the low bf16 parts lo = bf16(x - bf16(x)) of the tile-ordered keys and
 * values (and, with QK-norm + RoPE, queries).  The fine branch then forms
 * every product of fp32 operands a, b as a_hi*b_hi + a_hi*b_lo + a_lo*b_hi on
 * the bf16 matrix cores with fp32 sums, for q.k and for p.v alike, so its
 * result carries fp32-level error (about 2^-16 relative per product) instead
 * of bf16 rounding of the operands.  A VSA_F32 plan also runs bf16 forwards.
 * The workspace size changes: call before sizing and uploading a workspace.
 * VSA_E_ARG for another dtype. */
vsa_status vsa_h3_plan_set_io_dtype(vsa_h3_plan* plan, vsa_dtype io_dtype);

/* Host copies of the plan tables into caller-provided host buffers (any may
 * be NULL): perm int32 [Nt*tile_tokens], valid int32 [Nt] (tokens per tile),
 * tile_slot int32 [L] (tile*tile_tokens + slot of each packed token). */
vsa_status vsa_h3_plan_tables(const vsa_h3_plan* plan, int32_t* perm, int32_t* valid,
                              int32_t* tile_slot);

/* Copy the plan's tables into the workspace (device).  Must precede the first
 * vsa_h3_forward with this plan and workspace; they stay valid while the
 * caller does not overwrite that region. */
vsa_status vsa_h3_plan_upload(const vsa_h3_plan* plan, void* workspace,
                              uint64_t workspace_bytes, void* stream);

/* Enqueue the whole forward.
 *   q, k, v, gate  device [L][heads][head_dim] of io_dtype, read only.
 *   out            device [L][heads][head_dim] of io_dtype, fully written.
 *                  out = o_fine + gate * c[tile of the token], rounded to
 *                  io_dtype (nearest even).  Must not alias the inputs.
 *   sel_idx        device int32 [heads][NV][topk_ref + topk] or NULL;
 *                  receives the selected key tiles of each video query tile
 *                  (global tile ids, ascending: the selected reference tiles
 *                  when topk_ref > 0, then the selected video tiles).  NULL
 *                  keeps them in the workspace only.
 *   workspace      device, 256-byte aligned, >= workspace_bytes, holding the
 *                  tables from vsa_h3_plan_upload.  Calls that overlap in
 *                  time must use different workspaces.
 * Errors: VSA_E_ARG for NULL buffers, an unknown dtype or VSA_F32 on a plan
 * not set to it (vsa_h3_plan_set_io_dtype), VSA_E_WORKSPACE, VSA_E_HIP if a
 * launch fails (execution errors surface on the stream). */
vsa_status vsa_h3_forward(const vsa_h3_plan* plan, const void* q, const void* k, const void* v,
                          const void* gate, vsa_dtype io_dtype, void* out, int32_t* sel_idx,
                          void* workspace, uint64_t workspace_bytes, void* stream);

/* Same as vsa_h3_forward, and records caller-created HIP events (hipEvent_t,
 * passed as void*) on `stream` at the stage boundaries, for profiling tools:
 *   events[0] before the permute+pool kernel,
 *   events[1] after it (before the coarse-branch kernels),
 *   events[2] after the coarse branch (before the fine attention kernel),
 *   events[3] after the fine attention kernel.
 * `events` must point to 4 valid events; NULL behaves like vsa_h3_forward. */
vsa_status vsa_h3_forward_timed(const vsa_h3_plan* plan, const void* q, const void* k,
                                const void* v, const void* gate, vsa_dtype io_dtype, void* out,
                                int32_t* sel_idx, void* workspace, uint64_t workspace_bytes,
                                void* stream, void* const* events);

/* One-call form: builds (or reuses from an internal, thread-safe cache) the
 * plan for these tags / positions / grid / sizes / I/O dtype, uploads its
 * tables into the workspace and runs vsa_h3_forward.  Query the workspace
 * size first with vsa_h3_oneshot_workspace_bytes (same arguments). */
vsa_status vsa_h3_oneshot_workspace_bytes(const int64_t* token_tags, const int64_t* position_ids,
                                          int64_t L, vsa_dims3 grid, vsa_dims3 tile,
                                          int32_t heads, int32_t head_dim, double sparsity,
                                          vsa_dtype io_dtype, uint64_t* bytes_out);
vsa_status vsa_h3_forward_oneshot(const void* q, const void* k, const void* v, const void* gate,
                                  const int64_t* token_tags, const int64_t* position_ids,
                                  int64_t L, int32_t heads, int32_t head_dim, vsa_dims3 grid,
                                  double sparsity, vsa_dims3 tile, vsa_dtype io_dtype, void* out,
                                  int32_t* sel_idx, void* workspace, uint64_t workspace_bytes,
                                  void* stream);

/* Optional upstream step fused into the tile gather: QK RMS norm and RoPE
 * (FastH3 NVFP4 on RTX PRO 6000, "Model integration": QK-norm and RoPE are
 * applied to the tile-ordered q and k with cos/sin tables computed once per
 * step; pad rows stay zero).  The H3 norm weights and RoPE frequencies are
 * not published, so both are inputs.
 *
 * vsa_h3_plan_set_qk_prep(plan, 1) adds the workspace region that holds the
 * normalised, rotated q in tile order (the workspace size changes: call it
 * before sizing and uploading a workspace); 0 removes it.
 *
 * vsa_h3_forward_qk_prep runs the forward of vsa_h3_forward_timed on
 *   q' = rope(norm(q, q_norm_weight)),  k' = rope(norm(k, k_norm_weight)),
 * where, per (token, head) row x of head_dim D, in fp32 and in this order
 * (each operation separately rounded, no fused multiply-add):
 *   ss = sum_{d=0..D-1} x_d * x_d (sequential from +0);
 *   inv = 1 / sqrt(ss / D + eps)  (division, square root, reciprocal
 *         correctly rounded);
 *   y_d = (x_d * inv) * w_d;
 *   (y_2i, y_2i+1) -> (y_2i * c - y_2i+1 * s, y_2i * s + y_2i+1 * c) with
 *         c = rope_cos[token][i], s = rope_sin[token][i];
 * then rounded to io_dtype.  q', k' replace q, k everywhere (pooling,
 * scores, selection, fine branch); v and gate are used as given.
 *   q_norm_weight, k_norm_weight  device fp32 [head_dim], shared by all heads.
 *   eps                           finite, >= 0.
 *   rope_cos, rope_sin            device fp32 [L][head_dim/2], packed token order.
 *   events                        as for vsa_h3_forward_timed (may be NULL).
 * Errors: as vsa_h3_forward_timed; VSA_E_ARG if the plan has no QK-prep
 * region, a table or weight pointer is NULL or not 4-byte aligned, or eps
 * is negative or not finite. */
vsa_status vsa_h3_plan_set_qk_prep(vsa_h3_plan* plan, int32_t enable);
vsa_status vsa_h3_forward_qk_prep(const vsa_h3_plan* plan, const void* q, const void* k,
                                  const void* v, const void* gate, const float* q_norm_weight,
                                  const float* k_norm_weight, float eps, const float* rope_cos,
                                  const float* rope_sin, vsa_dtype io_dtype, void* out,
                                  int32_t* sel_idx, void* workspace, uint64_t workspace_bytes,
                                  void* stream, void* const* events);

/* Optional 8-bit Q/K in the fine branch (the OmniRef page, "Fallbacks":
 * per-token FP8 Q/K with bf16 P.V).  With vsa_h3_plan_set_qk_fp8(plan, 1)
 * every forward of this plan (vsa_h3_forward, _timed, _qk_prep) computes the
 * fine-branch logits from per-token OCP FP8 E4M3 q and k:
 *   for each (token, head) row x of q and of k: amax = max_d |x_d|;
 *   code_d = E4M3(x_d * (448 / amax)) (division correctly rounded, product
 *   rounded to fp32, E4M3 rounding to nearest even); scale = amax / 448;
 *   logit = scale_q * scale_k * sum_d decode(q_code_d) * decode(k_code_d) / sqrt(D).
 * Pooling, scores, selection, the coarse branch and P.V (bf16) are unchanged.
 * The workspace size changes (regions kt8 and kscale): call before sizing and
 * uploading a workspace; 0 switches back to bf16 q and k. */
vsa_status vsa_h3_plan_set_qk_fp8(vsa_h3_plan* plan, int32_t enable);

/* Reference keep ratio (the OmniRef page, "Device profiles": its Blackwell
 * stack keeps 0.1 of the reference tiles; the rule is not spelled out there).
 * With keep r < 1 every video query tile of every later forward of this plan
 * visits, among the prefix key tiles, the non-reference ones (text, audio)
 * and only the
 *     topk_ref = max(1, min(ceil(r * n_ref), n_ref))
 * reference (cond) tiles with the highest tile scores (ties to the lower
 * tile id; evaluated in IEEE double as written), next to its top-k video
 * tiles.  Prefix query tiles still visit every tile, and the compression
 * branch still covers every key tile.  r = 1 (the default) visits every
 * reference tile.  The workspace size changes (sel width and the visit
 * list): call before sizing and uploading a workspace.
 * VSA_E_ARG if r is outside (0, 1] or NaN. */
vsa_status vsa_h3_plan_set_ref_keep(vsa_h3_plan* plan, double keep);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * forward of vsa_h3_forward with the workspace taken from a device array
 * inside the library instead of from the caller.  It calls no hipMalloc,
 * hipFree or other allocating routine.
 *   - The array holds 64 MiB on every GPU the library runs on, from the
 *     first call on that GPU until the process ends.  A plan whose
 *     workspace_bytes exceeds 64 MiB is refused with VSA_E_WORKSPACE (for
 *     example the 480p 15,104-token layout fits at up to 7 heads).
 *   - The device is the current one (hipGetDevice); the first call on a
 *     device looks up that device's copy of the array.
 *   - Each call first copies the plan's tables into the array on `stream`
 *     (from host memory, as vsa_h3_plan_upload does), then runs the forward
 *     there; nothing else in the array needs clearing.
 *   - Every call on one GPU shares that GPU's array and leaves its contents
 *     behind: calls that overlap in time on one GPU (other streams, other
 *     threads) race and corrupt each other's results.  Serialize them.
 * Arguments, outputs and errors as for vsa_h3_forward. */
vsa_status vsa_h3_forward_noalloc(const vsa_h3_plan* plan, const void* q, const void* k,
                                  const void* v, const void* gate, vsa_dtype io_dtype, void* out,
                                  int32_t* sel_idx, void* stream);

void vsa_h3_plan_destroy(vsa_h3_plan* plan);
const char* vsa_h3_last_error(void);
const char* vsa_h3_version(void);

#ifdef __cplusplus
}
#endif
#endif /* VSA_H3_H */

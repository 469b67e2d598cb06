/*
 * ssta.h -- C ABI of the MI355X (gfx950) SSTA forward library, libssta.so.
 *
 * Selective and Sliding Tile Attention (SSTA) forward, as described on the
 * "HunyuanVideo 1.5 Technical Report" summary page, section "SSTA: Selective
 * and Sliding Tile Attention" (Steps 1-4), with the scoring details of the
 * importance_sampling excerpt on the "HunyuanVideo-1.5: An 8.3B-Parameter
 * Video Diffusion Model Built for Consumer GPUs" page, section "Under the
 * Hood: SSTA and Muon in Detail".
 *
 * Conventions shared by every entry point:
 *   - Tensors are device pointers, allocated and owned by the caller.  The
 *     library never allocates, frees or keeps device memory between calls.
 *   - Tensor pointers must be 16-byte aligned and densely packed in the
 *     layout stated for them.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  All
 *     device work is enqueued on it; no call synchronises the host.
 *   - Every call returns an ssta_status (0 = success).  Arguments are
 *     checked on the host before any HIP call, so a rejected call has
 *     enqueued nothing.  Faults inside kernels surface at the caller's next
 *     synchronisation.  There is no fallback path: if the current device is
 *     missing or is not gfx950 the call fails with SSTA_ERR_NO_DEVICE or
 *     SSTA_ERR_ARCH.
 *   - Tokens of a clip are numbered n = (t*H + y)*W + x.  Blocks ("tiles")
 *     are numbered row-major over the (T/tile_t, H/tile_h, W/tile_w) block
 *     grid, and the tokens of one block row-major over (tile_t, tile_h,
 *     tile_w).  n_tiles = (T/tile_t)(H/tile_h)(W/tile_w)  (Step 1).
 *   - Grids the block size does not divide are allowed: the block grid rounds
 *     up per axis and the blocks on the far edges hold only the tokens that
 *     exist (block means average those; attention runs over them; positions
 *     without a token are zero in tile-major copies and outputs and have LSE
 *     -inf).
 *   - Joint video + text sequences ("HunyuanVideo-1.5: An 8.3B-Parameter
 *     Video Diffusion Model Built for Consumer GPUs" page: section
 *     "Architecture: From Prompt to Video", single-stream blocks concatenate
 *     text and video tokens; section "Under the Hood: SSTA and Muon in
 *     Detail", text masking keeps the text out of scoring): with text_len > 0
 *     each (batch, head) holds S = T*H*W + text_len tokens, the clip's first.
 *     The text is cut into ceil(text_len/tile_tokens) blocks of consecutive
 *     tokens, numbered after the clip's n_tiles blocks: n_rows = n_tiles +
 *     text blocks (ssta_block_rows).  Only clip blocks are pooled, scored and
 *     selected; in attention every clip query block also keeps every text
 *     block and a text query block keeps every block.
 *   - Kept lists (kv_idx, kv_cnt) are inputs the kernels trust for their
 *     meaning: every row lists distinct clip block ids in [0, n_tiles),
 *     ascending, and kv_cnt is in [0, max_kept].  ssta_build_mask writes
 *     lists of that form.  For memory safety only, the attention kernels
 *     clamp each count to [0, max_kept] and each id to [0, n_tiles), and the
 *     backward ignores ids outside that range when it transposes the lists,
 *     so a malformed list never reads or writes outside the caller's
 *     buffers; its results are then unspecified.
 *   - Current limits: head_dim == 128, tile_t*tile_h*tile_w == 128 or 64 tokens;
 *     ssta_score_select and ssta_scores need n_tiles <= 4096 and
 *     batch*heads <= 65535;
 *     the attention entry points need n_rows < 65536 (one head's blocks are
 *     addressed with 32-bit offsets).
 */
#ifndef SSTA_H
#define SSTA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssta_status {
  SSTA_OK = 0,
  SSTA_ERR_ARG = -1,        /* null pointer, negative size, non-finite weight, unknown flag */
  SSTA_ERR_SHAPE = -2,      /* unsupported geometry (see limits above) or size overflow */
  SSTA_ERR_ALIGN = -3,      /* a tensor pointer is not 16-byte aligned */
  SSTA_ERR_NO_DEVICE = -4,  /* no HIP device is usable */
  SSTA_ERR_ARCH = -5,       /* the current device is not gfx950 */
  SSTA_ERR_HIP = -6,        /* a HIP launch failed; see ssta_last_hip_error() */
  SSTA_ERR_WORKSPACE = -7   /* workspace missing or smaller than ssta_workspace_bytes() */
} ssta_status;

/* Clip geometry.  All fields >= 1 except text_len. */
typedef struct ssta_geom {
  int32_t batch, heads, head_dim;   /* head_dim must be 128 */
  int32_t T, H, W;                  /* latent grid, tokens row-major (t, y, x) */
  int32_t tile_t, tile_h, tile_w;   /* block size; product 128 or 64 (so powers of two) */
  int32_t text_len;                 /* >= 0 text tokens after the clip's (0: clip only) */
} ssta_geom_t;

/* Selection and attention parameters. */
typedef struct ssta_params {
  int32_t win_t, win_h, win_w;  /* window half-widths in blocks (>= 0): a block j is in
                                   the window of block i when its block coordinates differ
                                   by at most these on every axis; clipped at the grid edge
                                   (Step 3, window size 2*half+1 per axis) */
  int32_t topk;                 /* >= 0; blocks selected per query block, clamped to the
                                   number of candidates (Step 2, Topk) */
  float lambda_, beta;          /* Score_i = lambda_*Score_s - beta*Score_r (Step 2);
                                   the excerpt's defaults are 0.9f and 0.1f */
  float scale;                  /* softmax scale, > 0; 1/sqrt(head_dim) in the attention
                                   equation */
  uint32_t flags;               /* SSTA_* flags below */
} ssta_params_t;

/*
 * Fills *p with the parameters the pages use: window half-widths (1, 1, 1),
 * topk 0 (set it to the number of blocks to select), lambda_ = 0.9f and
 * beta = 1 - lambda_ (the importance_sampling excerpt's weights: its 0.9
 * and 1 - 0.9 applied to fp32 scores act as the fp32 values 0.9f and 0.1f),
 * scale = 1/sqrt(head_dim) rounded to fp32 (the attention equation's
 * 1/sqrt(d_k)), no flags.  head_dim must be >= 1.
 * Returns SSTA_OK, or SSTA_ERR_ARG for a null pointer or head_dim < 1.
 */
int ssta_default_params(ssta_params_t* p, int32_t head_dim);

/* Step 4 prints the combination as a logical AND; the default is the union of
 * window and selection.  With this flag the kept set is their intersection
 * (a query block may then keep nothing: its output is 0 and its LSE -inf). */
#define SSTA_COMBINE_AND (1u << 0)
/* Select the top-k among the blocks outside the query block's window. */
#define SSTA_TOPK_EXCLUDE_WINDOW (1u << 1)

/* Layouts of a tiled tensor written by ssta_tile_pool. */
#define SSTA_LAYOUT_TOKEN_MAJOR 0   /* [batch, heads, n_rows, tile_tokens, head_dim] */
#define SSTA_LAYOUT_DIM_MAJOR 1     /* [batch, heads, n_rows, head_dim, tile_tokens] */

/* Blocks per (batch, head), n_rows: the clip's n_tiles plus
 * ceil(text_len / tile_tokens) text blocks.  < 0 on a bad argument. */
int64_t ssta_block_rows(const ssta_geom_t* g);

/*
 * Step 1 (3D block partition) and the block means of Step 2.
 *   x       in : bf16 [batch, heads, S, head_dim], token-major (S = T*H*W + text_len).
 *   x_tiled out: bf16, the same values gathered block by block in `layout`
 *                (SSTA_LAYOUT_*), clip blocks then text blocks; NULL to skip.
 *   pooled  out: fp32 [batch, heads, n_tiles, head_dim], the mean of each
 *                clip block's tokens: the fp32 sum over the block's existing
 *                tokens in ascending in-block order divided by their count;
 *                NULL to skip.  Text blocks have no mean.
 * Positions an edge block of a ragged grid lacks, and positions past the
 * text, are zero in x_tiled.  At least one of x_tiled and pooled must be
 * non-NULL.
 */
int ssta_tile_pool(const ssta_geom_t* g, const void* x, void* x_tiled, int32_t layout,
                   float* pooled, void* stream);

/*
 * Inverse of the token-major gather: x_tiled bf16 [batch, heads, n_rows,
 * tile_tokens, head_dim] -> x bf16 [batch, heads, S, head_dim].
 */
int ssta_tile_unpermute(const ssta_geom_t* g, const void* x_tiled, void* x, void* stream);

/* Width of each row of topk_idx: min(topk, n_tiles), or with
 * SSTA_TOPK_EXCLUDE_WINDOW min(topk, n_tiles - smallest window).  < 0 on a bad argument. */
int32_t ssta_topk_width(const ssta_geom_t* g, const ssta_params_t* p);

/* Row capacity of kv_idx: min(n_tiles, largest window + topk width), or with
 * SSTA_COMBINE_AND min(largest window, topk width).  < 0 on a bad argument. */
int32_t ssta_max_kept(const ssta_geom_t* g, const ssta_params_t* p);

/* Device workspace bytes that ssta_score_select and ssta_scores need.  < 0 on a bad argument. */
int64_t ssta_workspace_bytes(const ssta_geom_t* g, const ssta_params_t* p);

/*
 * Step 2 (selective mask): importance scores and per-query-block top-k.
 *   q_pooled, k_pooled in: fp32 [batch, heads, n_tiles, head_dim] block means.
 *   topk_idx out: int32 [batch, heads, n_tiles, ssta_topk_width()], the
 *                 selected key blocks of every query block in ascending id,
 *                 -1 padded when a row has fewer candidates than the width.
 *   workspace: device scratch of ws_bytes >= ssta_workspace_bytes().
 * Scores: qhat = q/|q|, khat = k/|k| (fp32, correctly rounded sqrt and
 * division; a zero vector stays zero); Score_s(i,j) = (qhat_i.khat_j+1)/2;
 * Score_r(j) = mean over key blocks i != j of (khat_i.khat_j+1)/2;
 * Score_i = lambda_*Score_s - beta*Score_r.  Every dot product is an fp32
 * fused-multiply-add chain in ascending channel order; the redundancy sum
 * adds, from +0, the terms of each group of 128 key blocks in ascending i,
 * then the group sums in ascending group order; nothing else is fused.  The
 * selection is thus a deterministic function of the inputs.  Ties go to the
 * lower block id.  The workspace holds qhat, khat, Score_r, its group sums
 * and the Score_i matrix (bh * n_tiles^2 floats) that the top-k reads.
 */
int ssta_score_select(const ssta_geom_t* g, const ssta_params_t* p, const float* q_pooled,
                      const float* k_pooled, int32_t* topk_idx, void* workspace,
                      size_t ws_bytes, void* stream);

/*
 * ssta_score_select without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc).  Same inputs, output and results as
 * ssta_score_select.  The scratch is a static device array of 64 MiB that
 * the library holds on every GPU it runs on until the process ends; the heads
 * are scored in groups that fit it.  Allocates nothing and calls no
 * allocating routine.
 *   Errors: as ssta_score_select (no SSTA_ERR_WORKSPACE), and SSTA_ERR_SHAPE
 *   when one head's scoring state (normalised means, Score_r and its group
 *   sums, the n_tiles^2 Score_i matrix: about n_tiles^2 * 4 bytes) exceeds
 *   the 64 MiB, i.e. beyond about 3,940 blocks per head.
 *   Every call on a GPU uses that GPU's one array: calls that overlap on one
 *   GPU (other streams, other host threads) race and give wrong ids;
 *   serialise them.  Nothing in the array needs to start at zero.
 */
int ssta_score_select_noalloc(const ssta_geom_t* g, const ssta_params_t* p,
                              const float* q_pooled, const float* k_pooled, int32_t* topk_idx,
                              void* stream);

/*
 * Inspection entry point for the same scoring: writes the full fp32
 * Score_i matrix scores [batch, heads, n_tiles, n_tiles] (row = query block)
 * and, if non-NULL, red [batch, heads, n_tiles] (Score_r).
 */
int ssta_scores(const ssta_geom_t* g, const ssta_params_t* p, const float* q_pooled,
                const float* k_pooled, float* scores, float* red, void* workspace,
                size_t ws_bytes, void* stream);

/*
 * Step 3 (sliding-tile window) and Step 4 (mask combination).
 *   topk_idx in : int32 [batch, heads, n_tiles, ssta_topk_width()] as written by
 *                 ssta_score_select (ascending, -1 padded).
 *   kv_idx  out : int32 [batch, heads, n_tiles, ssta_max_kept()], the kept key
 *                 blocks of each query block in ascending id, -1 padded.
 *   kv_cnt  out : int32 [batch, heads, n_tiles], number of kept blocks.
 *   bitmask out : uint32 [batch, heads, n_tiles, ceil(n_tiles/32)], bit j%32 of
 *                 word j/32 set iff block j is kept; NULL to skip.
 */
int ssta_build_mask(const ssta_geom_t* g, const ssta_params_t* p, const int32_t* topk_idx,
                    int32_t* kv_idx, int32_t* kv_cnt, uint32_t* bitmask, void* stream);

/*
 * Step 4 (block-sparse attention): for every query token of block i, softmax
 * of scale*q.k over the tokens of the kept key blocks of i only, then the
 * weighted sum of their values; full attention inside a kept block.  On a
 * joint sequence the kept blocks of a clip query block are its list plus
 * every text block, and a text query block keeps every block.
 *   q_t, k_t in : bf16 [batch, heads, n_rows, tile_tokens, head_dim] (token-major tiles).
 *   v_t      in : bf16 [batch, heads, n_rows, head_dim, tile_tokens] (dim-major tiles).
 *   kv_idx, kv_cnt in: as written by ssta_build_mask (clip blocks only);
 *                 kv_idx row stride max_kept (>= 1).  Pass kv_idx = kv_cnt =
 *                 NULL and max_kept = 0 for dense attention (every block kept).
 *   o_t     out : bf16 [batch, heads, n_rows, tile_tokens, head_dim] (token-major tiles).
 *   lse     out : fp32 [batch, heads, n_rows, tile_tokens], natural-log
 *                 log-sum-exp of the scaled scores; NULL to skip.
 * Arithmetic: bf16 products on the matrix cores, fp32 accumulation, fp32
 * online softmax.  A row with no kept block yields o = 0, lse = -inf.
 */
int ssta_attention_fwd(const ssta_geom_t* g, const ssta_params_t* p, const void* q_t,
                       const void* k_t, const void* v_t, const int32_t* kv_idx,
                       const int32_t* kv_cnt, int32_t max_kept, void* o_t, float* lse,
                       void* stream);

/*
 * Step 4 with the block gathers and the output scatter folded into the
 * attention kernel: the same computation as ssta_attention_fwd, but Q, K, V
 * and the output O stay in the caller's token order, so no input needs a
 * block copy and O no unpermute (each kept key block's K and V rows are
 * gathered token row by token row straight into LDS; the P.V product reads
 * its V^T operand from the token rows with transposing LDS loads).
 *   q        in : bf16 [batch, heads, S, head_dim] (token-major).
 *   k        in : bf16 [batch, heads, S, head_dim] (token-major).
 *   v        in : bf16 [batch, heads, S, head_dim] (token-major).
 *   kv_idx, kv_cnt, max_kept, lse: as for ssta_attention_fwd (LSE stays tile-major).
 *   o       out : bf16 [batch, heads, S, head_dim] (token-major).
 * Results are bit-identical to permuting Q, K (token-major tiles) and V
 * (dim-major tiles) with ssta_tile_pool, ssta_attention_fwd and
 * ssta_tile_unpermute.
 */
int ssta_attention_fwd_tokens(const ssta_geom_t* g, const ssta_params_t* p, const void* q,
                              const void* k, const void* v, const int32_t* kv_idx,
                              const int32_t* kv_cnt, int32_t max_kept, void* o, float* lse,
                              void* stream);

/* Device workspace bytes that ssta_attention_bwd needs.  < 0 on a bad argument. */
int64_t ssta_attention_bwd_workspace_bytes(const ssta_geom_t* g);

/*
 * Gradients of Step 4's block-sparse attention with the kept lists held fixed
 * ("HunyuanVideo 1.5 Technical Report" summary page, section "SSTA: Selective
 * and Sliding Tile Attention": the attention equation and Step 4; the same
 * section applies SSTA while the model is trained during distillation, so
 * gradients flow through the sparse attention; the block selection is an
 * integer and carries none).  For a query token a and the tokens b of its
 * kept blocks (on a joint sequence: as in the forward, text blocks always
 * kept, text query blocks keeping every block):
 * p_ab = exp(scale q_a.k_b - lse_a), D_a = dO_a.O_a,
 * dS_ab = p_ab (dO_a.v_b - D_a); dq_a = scale sum_b dS_ab k_b,
 * dk_b = scale sum_a dS_ab q_a, dv_b = sum_a p_ab dO_a.
 *   q, k, v, o, dout in : bf16 [batch, heads, S, head_dim] (token-major);
 *                         o and lse are the forward's outputs for these inputs.
 *   lse      in : fp32 [batch, heads, n_rows, tile_tokens] (tile-major, as the
 *                 forward writes it).  A query block that keeps nothing gets
 *                 dq = 0 and contributes to no dk, dv.
 *   kv_idx, kv_cnt, max_kept: the forward's kept lists (NULL, NULL, 0: dense).
 *   dq, dk, dv out : bf16 [batch, heads, S, head_dim] (token-major).
 *   workspace: device scratch of ws_bytes >= ssta_attention_bwd_workspace_bytes()
 *              (per-query (lse, D); the transposed lists and each head's key
 *              blocks ordered by how many query blocks keep them, which only
 *              schedules the dk/dv work).
 *              Caller-owned; contents on return are unspecified.
 * Probabilities and dS enter the matrix products as bf16, accumulation is fp32.
 * Errors: as ssta_attention_fwd, plus SSTA_ERR_WORKSPACE.
 */
int ssta_attention_bwd(const ssta_geom_t* g, const ssta_params_t* p, const void* q,
                       const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, const int32_t* kv_idx, const int32_t* kv_cnt,
                       int32_t max_kept, void* dq, void* dk, void* dv, void* workspace,
                       size_t ws_bytes, void* stream);

/* Measurement aid, not a step of the method.  For callers that want the
 * sustained bf16 matrix-core rate of the chip next to the attention kernel:
 * `grid` workgroups of 4 waves each run `iters` rounds of 4 independent
 * v_mfma_f32_32x32x16_bf16 products on register-resident operands read once
 * from `operands`.  The rate under random operands is what the power limit
 * allows for real data; constant operands draw less power.
 *   operands in : device, 256 x 8 bf16 (4 KB, 16-byte aligned).
 *   sink    out : device, grid*256 floats (keeps the work from being dropped).
 *   Work: grid * 4 * iters * 4 * 32768 FLOP.
 * Errors: SSTA_ERR_ARG for grid or iters <= 0 or null pointers, SSTA_ERR_ALIGN,
 * SSTA_ERR_NO_DEVICE / _ARCH, SSTA_ERR_HIP. */
int ssta_calibrate_mfma(const void* operands, float* sink, int32_t grid, int32_t iters,
                        void* stream);

/* Static text for a status code. */
const char* ssta_status_string(int status);

/* The hipError_t of the last SSTA_ERR_HIP on this thread (0 if none). */
int ssta_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SSTA_H */

/*
 * SSTA CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, sequential C for what the Selective and Sliding Tile Attention
 * (SSTA) forward computes.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or table with the GPU library.
 *
 * Sources (cited by page and section):
 *   [TR]   "HunyuanVideo 1.5 Technical Report" summary page, section
 *          "SSTA: Selective and Sliding Tile Attention": the attention
 *          equation, Step 1 (3D block partition, block count B), Step 2
 *          (Score_s, Score_r, Score_i, Topk, Indexes2mask), Step 3 (M_sta),
 *          Step 4 (mask combination, flex_block_attention).
 *   [BLOG] "HunyuanVideo-1.5: An 8.3B-Parameter Video Diffusion Model Built
 *          for Consumer GPUs", section "Under the Hood: SSTA and Muon in
 *          Detail": the importance_sampling code excerpt (cosine
 *          normalisation, (x+1)/2 map, diagonal-excluded mean redundancy,
 *          lambda = 0.9 with beta = 1 - lambda, top-k clamped to the block
 *          count, unsorted top-k).
 *
 * Floating-point rules (the pages fix no order; these are the readings):
 *   - scoring runs in fp32 with every operation written out: dot products
 *     are fmaf chains over the channel index in ascending order starting at
 *     0.0f; sqrtf and '/' are IEEE correctly rounded; nothing is contracted
 *     (compile with -ffp-contract=off);
 *   - tile means are fp32 sums over the in-tile token index in ascending
 *     order, divided by the token count;
 *   - attention uses the exact fp32 widening of the bf16 inputs, fp64
 *     accumulation and a two-pass softmax (max, then sum).
 *
 * Joint video + text sequences ([BLOG] section "Architecture: From Prompt to
 * Video": single-stream blocks concatenate text and video tokens; section
 * "Under the Hood: SSTA and Muon in Detail": the selection supports text
 * masking, so scoring skips the text tokens).  Readings: each (batch, head)
 * holds the N = T*H*W clip tokens followed by text_len text tokens; the
 * text is cut into blocks of tile_tokens consecutive tokens (the last one
 * partial) numbered after the clip's blocks; only clip blocks are pooled,
 * scored and selected; every clip query block also keeps every text block;
 * a text query block keeps every block.
 *
 * Parity pins: every function here is pinned by tests (closed forms,
 * brute force, library special cases); see the tests for each.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t batch, heads, head_dim;
  int32_t T, H, W;
  int32_t tile_t, tile_h, tile_w;
  int32_t text_len;   /* text tokens after the clip's tokens (joint sequence) */
} orc_geom;

enum { ORC_COMBINE_AND = 1u << 0, ORC_TOPK_EXCLUDE_WINDOW = 1u << 1 };

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Reading for grids the block size does not divide: the block grid rounds up
 * and the blocks on the far edges hold only the tokens that exist. */
static int64_t tiles_t(const orc_geom* g) { return (g->T + g->tile_t - 1) / g->tile_t; }
static int64_t tiles_h(const orc_geom* g) { return (g->H + g->tile_h - 1) / g->tile_h; }
static int64_t tiles_w(const orc_geom* g) { return (g->W + g->tile_w - 1) / g->tile_w; }

/* [TR] Step 1: block count = (F/tile_t)(H/tile_h)(W/tile_w), rounded up per axis. */
int64_t orc_n_tiles(const orc_geom* g) { return tiles_t(g) * tiles_h(g) * tiles_w(g); }

int32_t orc_tile_tokens(const orc_geom* g) { return g->tile_t * g->tile_h * g->tile_w; }

/* Tokens per (batch, head): the clip's, then the text's. */
static int64_t seq_len(const orc_geom* g) {
  return (int64_t)g->T * g->H * g->W + g->text_len;
}

/* Blocks per (batch, head): the clip's blocks, then ceil(text_len / tile_tokens) text blocks. */
int64_t orc_n_rows(const orc_geom* g) {
  const int64_t R = orc_tile_tokens(g);
  return orc_n_tiles(g) + (g->text_len + R - 1) / R;
}

/*
 * [TR] Step 1: tokens are grouped into contiguous 3D blocks.
 * Reading: blocks are numbered row-major over the (t, h, w) block grid and
 * tokens inside a block row-major over (t, h, w); token n = (t*H + y)*W + x.
 */
void orc_token_to_tile(const orc_geom* g, int64_t n, int64_t* tile, int32_t* r) {
  const int64_t t = n / ((int64_t)g->H * g->W);
  const int64_t y = (n / g->W) % g->H;
  const int64_t x = n % g->W;
  *tile = ((t / g->tile_t) * tiles_h(g) + (y / g->tile_h)) * tiles_w(g) + (x / g->tile_w);
  *r = (int32_t)(((t % g->tile_t) * g->tile_h + (y % g->tile_h)) * g->tile_w + (x % g->tile_w));
}

/* Inverse map: the token index of in-tile position r of tile `tile`, or -1
 * when that position lies beyond the grid (an edge block of a ragged grid).
 * Blocks from n_tiles on are text blocks: position r of text block u is text
 * token u*tile_tokens + r, i.e. token N + u*tile_tokens + r (-1 past the text). */
int64_t orc_tile_to_token(const orc_geom* g, int64_t tile, int32_t r) {
  const int64_t n_clip = orc_n_tiles(g);
  if (tile >= n_clip) {
    const int64_t u = (tile - n_clip) * orc_tile_tokens(g) + r;
    return u < g->text_len ? (int64_t)g->T * g->H * g->W + u : -1;
  }
  const int64_t bt = tile / (tiles_h(g) * tiles_w(g));
  const int64_t by = (tile / tiles_w(g)) % tiles_h(g);
  const int64_t bx = tile % tiles_w(g);
  const int64_t it = r / (g->tile_h * g->tile_w);
  const int64_t iy = (r / g->tile_w) % g->tile_h;
  const int64_t ix = r % g->tile_w;
  const int64_t t = bt * g->tile_t + it, y = by * g->tile_h + iy, x = bx * g->tile_w + ix;
  if (t >= g->T || y >= g->H || x >= g->W) return -1;
  return (t * g->H + y) * g->W + x;
}

/* Gather x[b,h,S,D] (bf16 bits; S = N + text_len) into tile-major
 * x_t[b,h,n_rows,tile_tokens,D], clip blocks then text blocks; positions
 * beyond a ragged grid or past the text are zero. */
void orc_permute(const orc_geom* g, const uint16_t* x, uint16_t* x_t) {
  const int64_t N = (int64_t)g->T * g->H * g->W, S = seq_len(g), D = g->head_dim;
  const int64_t BH = (int64_t)g->batch * g->heads, NR = orc_n_rows(g);
  const int64_t R = orc_tile_tokens(g);
  memset(x_t, 0, sizeof(uint16_t) * (size_t)(BH * NR * R * D));
  for (int64_t bh = 0; bh < BH; ++bh)
    for (int64_t n = 0; n < S; ++n) {
      int64_t tile;
      int32_t r;
      if (n < N) {
        orc_token_to_tile(g, n, &tile, &r);
      } else {
        tile = orc_n_tiles(g) + (n - N) / R;
        r = (int32_t)((n - N) % R);
      }
      memcpy(x_t + ((bh * NR + tile) * R + r) * D, x + (bh * S + n) * D,
             (size_t)D * sizeof(uint16_t));
    }
}

/*
 * [TR] Step 2: pooled (average) block representation.
 * pooled[b,h,i,d] = (sum over the block's existing positions r, ascending, in
 * fp32, of x[token(i, r), d]) / (number of those positions): every position
 * of an interior block, the positions inside the grid for an edge block of a
 * ragged grid.
 */
void orc_pool(const orc_geom* g, const uint16_t* x, float* pooled) {
  const int64_t S = seq_len(g), D = g->head_dim;   /* text tokens are not pooled */
  const int64_t BH = (int64_t)g->batch * g->heads, NT = orc_n_tiles(g);
  const int32_t R = orc_tile_tokens(g);
#pragma omp parallel for schedule(static)
  for (int64_t bhi = 0; bhi < BH * NT; ++bhi) {
    const int64_t bh = bhi / NT, i = bhi % NT;
    float s[1024];
    int32_t count = 0;
    for (int64_t d = 0; d < D; ++d) s[d] = 0.0f;
    for (int32_t r = 0; r < R; ++r) {
      const int64_t tok = orc_tile_to_token(g, i, r);
      if (tok < 0) continue;
      ++count;
      const uint16_t* row = x + (bh * S + tok) * D;
      for (int64_t d = 0; d < D; ++d) s[d] = s[d] + bf16_to_f32(row[d]);
    }
    for (int64_t d = 0; d < D; ++d) pooled[bhi * D + d] = s[d] / (float)count;
  }
}

/*
 * [BLOG] importance_sampling: each pooled vector is divided by its L2 norm.
 * ss = fmaf chain of p[d]*p[d] over ascending d; nrm = sqrtf(ss);
 * out[d] = p[d] / nrm.  Reading: a zero vector stays zero (the pages do
 * not cover it; the excerpt would produce NaN).
 */
void orc_normalize(int64_t rows, int32_t D, const float* p, float* out) {
  for (int64_t i = 0; i < rows; ++i) {
    const float* v = p + i * D;
    float ss = 0.0f;
    for (int32_t d = 0; d < D; ++d) ss = fmaf(v[d], v[d], ss);
    const float nrm = sqrtf(ss);
    for (int32_t d = 0; d < D; ++d) out[i * D + d] = (nrm == 0.0f) ? 0.0f : v[d] / nrm;
  }
}

static float dot_f32(const float* a, const float* b, int32_t D) {
  float s = 0.0f;
  for (int32_t d = 0; d < D; ++d) s = fmaf(a[d], b[d], s);
  return s;
}

/*
 * [TR] Step 2, Score_r; [BLOG] gate_unique with the diagonal removed and a
 * mean over the remaining key blocks.
 * u(i, j) = (khat_i . khat_j + 1) * 0.5;
 * red[j] = (sum over the groups G = [128g, 128g + 128) of key blocks, in
 *           ascending g, of (sum over i in G, i != j, ascending i, fp32,
 *           starting from 0, of u(i, j))) / (n - 1);
 * red = 0 when n == 1.  Readings: the normaliser counts key blocks (n - 1);
 * the summary page's "N - 1" reuses the letter it gave the block size.  The
 * pages' mean over the other key blocks leaves the order of the sum open;
 * this two-level order (a partial sum per group of 128 key blocks, the
 * partials added in ascending group order) is fixed here because the
 * selection must be reproducible bit for bit.  With n <= 128 it is the plain
 * ascending sum.
 */
enum { RED_GROUP = 128 };
void orc_redundancy(int64_t BH, int64_t n, int32_t D, const float* khat, float* red) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t bhj = 0; bhj < BH * n; ++bhj) {
    const int64_t bh = bhj / n, j = bhj % n;
    const float* kb = khat + bh * n * D;
    float s = 0.0f;
    for (int64_t g0 = 0; g0 < n; g0 += RED_GROUP) {
      float part = 0.0f;
      for (int64_t i = g0; i < n && i < g0 + RED_GROUP; ++i) {
        if (i == j) continue;
        const float u = (dot_f32(kb + i * D, kb + j * D, D) + 1.0f) * 0.5f;
        part = part + u;
      }
      s = s + part;
    }
    red[bhj] = (n > 1) ? s / (float)(n - 1) : 0.0f;
  }
}

/*
 * [TR] Step 2, Score_s and Score_i; [BLOG] gate_similarity and
 * importance_scores.
 * g(i, j) = (qhat_i . khat_j + 1) * 0.5;
 * score(i, j) = (lambda * g(i, j)) - (beta * red[j]), two rounded products
 * and one rounded difference.
 */
void orc_scores(int64_t BH, int64_t n, int32_t D, const float* qhat, const float* khat,
                const float* red, float lambda_, float beta, float* scores) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t bhi = 0; bhi < BH * n; ++bhi) {
    const int64_t bh = bhi / n;
    const float* q = qhat + bhi * D;
    for (int64_t j = 0; j < n; ++j) {
      const float gs = (dot_f32(q, khat + (bh * n + j) * D, D) + 1.0f) * 0.5f;
      const float a = lambda_ * gs;
      const float b = beta * red[bh * n + j];
      scores[bhi * n + j] = a - b;
    }
  }
}

/* [TR] Step 3: the sliding-tile window.  WS = 2*half + 1 blocks per axis,
 * centred on the query block.  Reading: clipped at the grid edge (no wrap,
 * no shift).  Writes the window's block ids in ascending order; returns the
 * count. */
int32_t orc_window(const orc_geom* g, int32_t wt, int32_t wh, int32_t ww, int64_t i, int32_t* out) {
  const int64_t nt = tiles_t(g), ny = tiles_h(g), nx = tiles_w(g);
  const int64_t ti = i / (ny * nx), yi = (i / nx) % ny, xi = i % nx;
  int32_t c = 0;
  for (int64_t t = 0; t < nt; ++t) {
    if (llabs(t - ti) > wt) continue;
    for (int64_t y = 0; y < ny; ++y) {
      if (llabs(y - yi) > wh) continue;
      for (int64_t x = 0; x < nx; ++x) {
        if (llabs(x - xi) > ww) continue;
        out[c++] = (int32_t)((t * ny + y) * nx + x);
      }
    }
  }
  return c;
}

typedef struct { float s; int32_t j; } scored;

/* Higher score first; equal scores (IEEE ==, so -0 == +0): lower block id first. */
static int cmp_scored(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int cmp_i32(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/*
 * [TR] Step 2, Topk; [BLOG] topk clamped to the number of key blocks.
 * For each query-block row: sort all n candidates by (score descending,
 * block id ascending) and keep the first k_eff; output in ascending block
 * id (the pages leave the order unspecified).  With exclude_window != 0,
 * window blocks of the row (given per row by `geom`/win) are not
 * candidates.  idx_out has room for k_out entries per row; rows with fewer
 * candidates are padded with -1.  Returns 0, or -1 on a bad argument.
 */
int orc_topk(const orc_geom* g, int32_t wt, int32_t wh, int32_t ww, int32_t exclude_window,
             int64_t BH, int64_t n, const float* scores, int32_t k, int32_t k_out,
             int32_t* idx_out) {
  if (k < 0 || k_out < 0) return -1;
  int failed = 0;
#pragma omp parallel
  {
    scored* buf = (scored*)malloc(sizeof(scored) * (size_t)(n > 0 ? n : 1));
    int32_t* win = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    char* inwin = (char*)calloc((size_t)(n > 0 ? n : 1), 1);
    if (!buf || !win || !inwin) failed = 1;
#pragma omp for schedule(dynamic, 16)
    for (int64_t row = 0; row < BH * n; ++row) {
      if (failed) continue;
      const int64_t i = row % n;
      int32_t nw = 0;
      if (exclude_window) {
        nw = orc_window(g, wt, wh, ww, i, win);
        for (int32_t a = 0; a < nw; ++a) inwin[win[a]] = 1;
      }
      int64_t m = 0;
      for (int64_t j = 0; j < n; ++j) {
        if (exclude_window && inwin[j]) continue;
        buf[m].s = scores[row * n + j];
        buf[m].j = (int32_t)j;
        ++m;
      }
      if (exclude_window)
        for (int32_t a = 0; a < nw; ++a) inwin[win[a]] = 0;
      qsort(buf, (size_t)m, sizeof(scored), cmp_scored);
      int64_t keep = k < m ? k : m;
      if (keep > k_out) keep = k_out;
      int32_t* o = idx_out + row * (int64_t)k_out;
      for (int64_t a = 0; a < keep; ++a) o[a] = buf[a].j;
      qsort(o, (size_t)keep, sizeof(int32_t), cmp_i32);
      for (int64_t a = keep; a < k_out; ++a) o[a] = -1;
    }
    free(buf);
    free(win);
    free(inwin);
  }
  return failed ? -1 : 0;
}

/*
 * [TR] Step 4: combine the per-head selected blocks with the shared window.
 * Reading: union (ORC_COMBINE_AND gives the intersection that Algorithm 1
 * prints).  kv_idx rows are ascending and padded with -1 to max_kept;
 * kv_cnt holds the row length.  bitmask (nullable) gets bit j%32 of word
 * j/32 set for every kept block j, words per row = ceil(n/32).
 * Returns 0, or -1 if a row would exceed max_kept.
 */
int orc_build_lists(const orc_geom* g, int32_t wt, int32_t wh, int32_t ww, uint32_t flags,
                    const int32_t* topk_idx, int32_t k_stride, int32_t max_kept,
                    int32_t* kv_idx, int32_t* kv_cnt, uint32_t* bitmask) {
  const int64_t n = orc_n_tiles(g), BH = (int64_t)g->batch * g->heads;
  const int64_t words = (n + 31) / 32;
  int bad = 0;
  char* mark = (char*)calloc((size_t)n, 1);
  char* wmark = (char*)calloc((size_t)n, 1);
  int32_t* win = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  if (!mark || !wmark || !win) { free(mark); free(wmark); free(win); return -1; }
  for (int64_t row = 0; row < BH * n; ++row) {
    const int64_t i = row % n;
    const int32_t nw = orc_window(g, wt, wh, ww, i, win);
    for (int32_t a = 0; a < nw; ++a) wmark[win[a]] = 1;
    for (int32_t a = 0; a < k_stride; ++a) {
      const int32_t j = topk_idx[row * k_stride + a];
      if (j < 0) continue;
      if (flags & ORC_COMBINE_AND) { if (wmark[j]) mark[j] = 1; }
      else mark[j] = 1;
    }
    if (!(flags & ORC_COMBINE_AND))
      for (int32_t a = 0; a < nw; ++a) mark[win[a]] = 1;
    int32_t c = 0;
    for (int64_t j = 0; j < n; ++j) {
      if (!mark[j]) continue;
      if (c >= max_kept) { bad = 1; break; }
      kv_idx[row * max_kept + c++] = (int32_t)j;
    }
    for (int32_t a = c; a < max_kept; ++a) kv_idx[row * max_kept + a] = -1;
    kv_cnt[row] = c;
    if (bitmask) {
      uint32_t* bm = bitmask + row * words;
      for (int64_t w = 0; w < words; ++w) bm[w] = 0;
      for (int64_t j = 0; j < n; ++j)
        if (mark[j]) bm[j / 32] |= 1u << (j % 32);
    }
    for (int64_t j = 0; j < n; ++j) { mark[j] = 0; wmark[j] = 0; }
    if (bad) break;
  }
  free(mark);
  free(wmark);
  free(win);
  return bad ? -1 : 0;
}

/*
 * The key tokens of query block i of head bh ([TR] Step 4: the tokens of the
 * kept blocks; on a joint sequence also every text block, and every block
 * for a text query block).  Blocks in list order -- a clip row's kept list,
 * then the text blocks; a text row's blocks 0 .. n_rows-1 -- and tokens in
 * in-block order, positions without a token skipped.  blk[t] and pos[t] are
 * the block and in-block position of keys[t].
 */
static int64_t row_keys(const orc_geom* g, int64_t bh, int64_t i, const int32_t* kv_idx,
                        const int32_t* kv_cnt, int32_t max_kept, int64_t* keys, int64_t* blk,
                        int32_t* pos) {
  const int64_t n = orc_n_tiles(g), NR = orc_n_rows(g);
  const int32_t R = orc_tile_tokens(g);
  const int64_t clip_row = bh * n + i;
  const int64_t listed = i < n ? kv_cnt[clip_row] : 0;
  const int64_t nb = i < n ? listed + (NR - n) : NR;
  int64_t m = 0;
  for (int64_t c = 0; c < nb; ++c) {
    int64_t j;
    if (i >= n)
      j = c;                                    /* text query block: every block */
    else if (c < listed)
      j = kv_idx[clip_row * max_kept + c];      /* the kept clip blocks */
    else
      j = n + (c - listed);                     /* the text blocks, always kept */
    for (int32_t rr = 0; rr < R; ++rr) {
      const int64_t tok = orc_tile_to_token(g, j, rr);
      if (tok < 0) continue;
      keys[m] = tok;
      blk[m] = j;
      pos[m] = rr;
      ++m;
    }
  }
  return m;
}

/*
 * [TR] the attention equation and Step 4 (flex_block_attention): softmax of
 * scale * q.k over the keys of the kept blocks only, then the weighted sum
 * of their values; full attention inside a kept block (Step 1).
 * For each selected row (b*heads + h)*n_rows + i (n_rows = n_tiles without
 * text), writes o[sel][r][d] for the query at in-block position r (fp64) and
 * lse[sel][r] = log sum exp.  Inputs are token-major bf16 bits [b, h, S, D].
 * An empty key set, or a position without a token, gives o = 0 and lse = -inf.
 */
void orc_attention(const orc_geom* g, double scale, const uint16_t* q, const uint16_t* k,
                   const uint16_t* v, const int32_t* kv_idx, const int32_t* kv_cnt,
                   int32_t max_kept, int64_t n_sel, const int64_t* sel_rows, double* o_out,
                   double* lse_out) {
  const int64_t S = seq_len(g), D = g->head_dim, NR = orc_n_rows(g);
  const int32_t R = orc_tile_tokens(g);
  const size_t cap = (size_t)NR * R + 8;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * cap);
    double* qv = (double*)malloc(sizeof(double) * (size_t)D);
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * cap);
    int64_t* blk = (int64_t*)malloc(sizeof(int64_t) * cap);
    int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * cap);
#pragma omp for schedule(dynamic, 1)
    for (int64_t a = 0; a < n_sel; ++a) {
      const int64_t row = sel_rows[a], bh = row / NR, i = row % NR;
      const int64_t m = row_keys(g, bh, i, kv_idx, kv_cnt, max_kept, keys, blk, pos);
      for (int32_t r = 0; r < R; ++r) {
        const int64_t nq = orc_tile_to_token(g, i, r);
        double* o = o_out + (a * R + r) * D;
        for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
        if (m == 0 || nq < 0) { lse_out[a * R + r] = -INFINITY; continue; }
        for (int64_t d = 0; d < D; ++d) qv[d] = (double)bf16_to_f32(q[(bh * S + nq) * D + d]);
        double mx = -INFINITY;
        for (int64_t t = 0; t < m; ++t) {
          const uint16_t* kr = k + (bh * S + keys[t]) * D;
          double acc = 0.0;
          for (int64_t d = 0; d < D; ++d) acc += qv[d] * (double)bf16_to_f32(kr[d]);
          s[t] = acc * scale;
          if (s[t] > mx) mx = s[t];
        }
        double l = 0.0;
        for (int64_t t = 0; t < m; ++t) {
          s[t] = exp(s[t] - mx);
          l += s[t];
        }
        for (int64_t t = 0; t < m; ++t) {
          const uint16_t* vr = v + (bh * S + keys[t]) * D;
          const double p = s[t] / l;
          for (int64_t d = 0; d < D; ++d) o[d] += p * (double)bf16_to_f32(vr[d]);
        }
        lse_out[a * R + r] = mx + log(l);
      }
    }
    free(s);
    free(qv);
    free(keys);
    free(blk);
    free(pos);
  }
}

/*
 * Gradients of the block-sparse attention of Step 4 ([TR] "SSTA: Selective and
 * Sliding Tile Attention", the attention equation and Step 4; the same section's
 * paragraph on parameter-free integration: SSTA is applied while the model is
 * trained during distillation, so gradients flow through the sparse attention
 * with the kept lists held fixed -- the selection is an integer and carries none).
 *
 * For a query token a of block i with key tokens b (row_keys):
 * s_ab = scale q_a.k_b,  p_ab = softmax_b(s_ab),  o_a = sum_b p_ab v_b.  Given dO:
 *   D_a   = dO_a . o_a
 *   dS_ab = p_ab (dO_a . v_b - D_a)
 *   dq_a  = scale sum_b dS_ab k_b
 *   dk_b  = scale sum_a dS_ab q_a      (over every query token a whose keys hold b)
 *   dv_b  = sum_a p_ab dO_a
 * Everything in fp64 from the exact widening of the bf16 inputs.
 * dq is returned for the query-block rows q_rows, dk and dv for the key-block
 * rows k_rows (flat ids (b*heads + h)*n_rows + block), in in-block token order.
 */

/* Softmax row of query token (bh, nq) over the key tokens keys[0..m): p (m), o (D), D_a. */
static void bwd_row(const orc_geom* g, double scale, int64_t bh, int64_t nq, const uint16_t* q,
                    const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                    const int64_t* keys, int64_t m, double* qv, double* dov, double* p,
                    double* o, double* dsum) {
  const int64_t S = seq_len(g), D = g->head_dim;
  for (int64_t d = 0; d < D; ++d) {
    qv[d] = (double)bf16_to_f32(q[(bh * S + nq) * D + d]);
    dov[d] = (double)bf16_to_f32(dout[(bh * S + nq) * D + d]);
    o[d] = 0.0;
  }
  double mx = -INFINITY;
  for (int64_t t = 0; t < m; ++t) {
    const uint16_t* kr = k + (bh * S + keys[t]) * D;
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d) acc += qv[d] * (double)bf16_to_f32(kr[d]);
    p[t] = acc * scale;
    if (p[t] > mx) mx = p[t];
  }
  double l = 0.0;
  for (int64_t t = 0; t < m; ++t) {
    p[t] = exp(p[t] - mx);
    l += p[t];
  }
  for (int64_t t = 0; t < m; ++t) {
    p[t] /= l;
    const uint16_t* vr = v + (bh * S + keys[t]) * D;
    for (int64_t d = 0; d < D; ++d) o[d] += p[t] * (double)bf16_to_f32(vr[d]);
  }
  double da = 0.0;
  for (int64_t d = 0; d < D; ++d) da += dov[d] * o[d];
  *dsum = da;
}

/* dS_ab for the row (p holds the probabilities, overwritten with dS). */
static void bwd_ds(const orc_geom* g, int64_t bh, const uint16_t* v, const int64_t* keys,
                   int64_t m, const double* dov, double da, double* p) {
  const int64_t S = seq_len(g), D = g->head_dim;
  for (int64_t t = 0; t < m; ++t) {
    const uint16_t* vr = v + (bh * S + keys[t]) * D;
    double dp = 0.0;
    for (int64_t d = 0; d < D; ++d) dp += dov[d] * (double)bf16_to_f32(vr[d]);
    p[t] = p[t] * (dp - da);
  }
}

void orc_attention_bwd(const orc_geom* g, double scale, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, const uint16_t* dout, const int32_t* kv_idx,
                       const int32_t* kv_cnt, int32_t max_kept, int64_t n_qrows,
                       const int64_t* q_rows, double* dq_out, int64_t n_krows,
                       const int64_t* k_rows, double* dk_out, double* dv_out) {
  const int64_t S = seq_len(g), D = g->head_dim, NR = orc_n_rows(g);
  const int32_t R = orc_tile_tokens(g);
  const size_t cap = (size_t)NR * R + 8;
#pragma omp parallel
  {
    double* p = (double*)malloc(sizeof(double) * cap);
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * cap);
    int64_t* blk = (int64_t*)malloc(sizeof(int64_t) * cap);
    int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * cap);
    double* qv = (double*)malloc(sizeof(double) * (size_t)D);
    double* dov = (double*)malloc(sizeof(double) * (size_t)D);
    double* o = (double*)malloc(sizeof(double) * (size_t)D);
    /* dq: one selected query-block row per iteration */
#pragma omp for schedule(dynamic, 1)
    for (int64_t a = 0; a < n_qrows; ++a) {
      const int64_t row = q_rows[a], bh = row / NR, i = row % NR;
      const int64_t m = row_keys(g, bh, i, kv_idx, kv_cnt, max_kept, keys, blk, pos);
      for (int32_t r = 0; r < R; ++r) {
        double* dq = dq_out + (a * R + r) * D;
        for (int64_t d = 0; d < D; ++d) dq[d] = 0.0;
        const int64_t nq = orc_tile_to_token(g, i, r);
        if (m == 0 || nq < 0) continue;
        double da;
        bwd_row(g, scale, bh, nq, q, k, v, dout, keys, m, qv, dov, p, o, &da);
        bwd_ds(g, bh, v, keys, m, dov, da, p);
        for (int64_t t = 0; t < m; ++t) {
          const uint16_t* kr = k + (bh * S + keys[t]) * D;
          for (int64_t d = 0; d < D; ++d) dq[d] += scale * p[t] * (double)bf16_to_f32(kr[d]);
        }
      }
    }
    /* dk, dv: one selected key-block row per iteration; every query block of
       the head whose keys hold it contributes, in ascending block order */
#pragma omp for schedule(dynamic, 1)
    for (int64_t a = 0; a < n_krows; ++a) {
      const int64_t krow = k_rows[a], bh = krow / NR, j = krow % NR;
      double* dk = dk_out + a * R * D;
      double* dv = dv_out + a * R * D;
      for (int64_t e = 0; e < (int64_t)R * D; ++e) dk[e] = dv[e] = 0.0;
      for (int64_t i = 0; i < NR; ++i) {
        const int64_t m = row_keys(g, bh, i, kv_idx, kv_cnt, max_kept, keys, blk, pos);
        int found = 0;
        for (int64_t t = 0; t < m && !found; ++t) found = blk[t] == j;
        if (!found) continue;
        for (int32_t r = 0; r < R; ++r) {
          const int64_t nq = orc_tile_to_token(g, i, r);
          if (nq < 0) continue;
          double da;
          bwd_row(g, scale, bh, nq, q, k, v, dout, keys, m, qv, dov, p, o, &da);
          /* keep p for dv before it becomes dS */
          for (int64_t t = 0; t < m; ++t) {
            if (blk[t] != j) continue;
            for (int64_t d = 0; d < D; ++d) dv[pos[t] * D + d] += p[t] * dov[d];
          }
          bwd_ds(g, bh, v, keys, m, dov, da, p);
          for (int64_t t = 0; t < m; ++t) {
            if (blk[t] != j) continue;
            for (int64_t d = 0; d < D; ++d) dk[pos[t] * D + d] += scale * p[t] * qv[d];
          }
        }
      }
    }
    free(p);
    free(keys);
    free(blk);
    free(pos);
    free(qv);
    free(dov);
    free(o);
  }
}

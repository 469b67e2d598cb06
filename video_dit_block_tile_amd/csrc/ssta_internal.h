// Internal declarations shared by the host dispatcher (ssta_api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssta {

constexpr int kHeadDim = 128;     // channels per head
constexpr int kTileTokens = 128;  // tokens per 3D block (the default 2x8x8 block)
constexpr int kSmallTile = 64;    // tokens per block of the smaller shape (e.g. 4x4x4)
constexpr int kMaxTopkTiles = 4096;
constexpr int64_t kMaxScoreHeads = 65535;   // batch*heads of the scoring grids

// Geometry with every derived quantity precomputed on the host.
struct Geo {
  int32_t batch, heads, D;
  int32_t T, H, W;
  int32_t tt, th, tw;       // block size
  int32_t R;                // tokens per block: 128 or 64
  int32_t nt, ny, nx;       // block grid
  int64_t N;                // tokens per (batch, head)
  int64_t n_tiles;          // blocks per (batch, head)
  int64_t bh;               // batch * heads
  int32_t ragged;           // some axis is not a multiple of its block size: the blocks on
                            // the far edges of that axis hold fewer tokens
  int32_t L;                // text tokens after the clip's N (joint sequence)
  int32_t n_txt;            // text blocks: ceil(L / R), numbered from n_tiles on
  int64_t S;                // tokens per (batch, head): N + L
  int64_t n_rows;           // blocks per (batch, head): n_tiles + n_txt
};

// Grid of the attention kernels (forward and backward): first one workgroup
// per (batch*head, text block) of a joint sequence -- each runs over every
// block, many times a clip block's work -- dealt round-robin over the XCDs so
// they overlap everything else; then the clip blocks in head-synchronous XCD
// slices: XCD x takes, head after head, positions [x*slice, (x+1)*slice) of
// the head's blocks in a visiting order.  The text part is padded to a
// multiple of 8 workgroups so every slice keeps its XCD (the hardware deals
// workgroup ids round-robin over the 8 XCDs).  The visiting order is the
// block ids themselves, or, with 64-token blocks, groups of tt frame rows of
// blocks, each walked in tiles of tt x ty x tx blocks (row-major over the
// tiles, then inside each tile in (t, y, x) order), so that the workgroups
// an XCD runs at once cover a compact 3D patch whose windows share more key
// blocks in its L2.
struct AttnGrid {
  int64_t text_wgs;   // workgroups of the text blocks (multiple of 8)
  int64_t slice;      // clip blocks per XCD per head
  int64_t blocks;     // total workgroups
  int32_t tt, ty, tx; // tile of the visiting order (tx = 0: block id order)
};
inline AttnGrid attn_grid(const Geo& g) {
  AttnGrid a;
  a.text_wgs = (g.bh * g.n_txt + 7) / 8 * 8;
  a.slice = (g.n_tiles + 7) / 8;
  a.blocks = a.text_wgs + g.bh * a.slice * 8;
  a.tt = a.ty = a.tx = 0;
  if (g.R == kSmallTile) {
    a.tt = g.nt < 4 ? g.nt : 4;
    a.ty = g.ny < 2 ? g.ny : 2;
    a.tx = g.nx < 2 ? g.nx : 2;
  }
  return a;
}
// Block at position pos of the visiting order (a bijection on [0, n_tiles)):
// frame-row group f = pos / (tt*ny*nx) of ht rows (the last group possibly
// fewer); in it, rows of tiles ty high (the last possibly lower), tiles tx
// wide (the last possibly narrower), each tile in (t, y, x) order.
__device__ __forceinline__ int64_t visit_block(const Geo& g, const AttnGrid& a, int64_t pos) {
  if (a.tx == 0) return pos;
  const int64_t nyx = (int64_t)g.ny * g.nx;
  const int64_t f = pos / (a.tt * nyx), r = pos - f * a.tt * nyx;
  const int64_t ht = min((int64_t)a.tt, g.nt - f * a.tt);
  const int64_t row = r / (ht * a.ty * g.nx), rr = r - row * ht * a.ty * g.nx;
  const int64_t hy = min((int64_t)a.ty, g.ny - row * a.ty);
  const int64_t col = rr / (ht * hy * a.tx), off = rr - col * ht * hy * a.tx;
  const int64_t wx = min((int64_t)a.tx, g.nx - col * a.tx);
  const int64_t ti = off / (hy * wx), rem = off - ti * hy * wx;
  const int64_t yi = rem / wx, xi = rem - yi * wx;
  return (f * a.tt + ti) * nyx + (row * a.ty + yi) * g.nx + col * a.tx + xi;
}
// (batch*head, block) of workgroup bid; false for the padding workgroups.
// kText = false: the instance for sequences without text (text_wgs == 0).
template <bool kText>
__device__ __forceinline__ bool attn_block(const Geo& g, const AttnGrid& a, int64_t bid,
                                           int64_t& bh, int64_t& blk) {
  if (kText && bid < a.text_wgs) {
    bh = bid / g.n_txt;
    blk = g.n_tiles + bid % g.n_txt;
    return bh < g.bh;
  }
  const int64_t b = bid - a.text_wgs, xcd = b & 7, k8 = b >> 3;
  bh = k8 / a.slice;
  const int64_t pos = xcd * a.slice + (k8 - bh * a.slice);
  if (pos >= g.n_tiles) return false;
  blk = visit_block(g, a, pos);
  return true;
}

// Extent of block `tile` along each axis: the block size, except at the far
// edges of a ragged grid.
struct BlockExtent {
  int32_t lt, ly, lx;
  bool full;
};
__device__ __forceinline__ BlockExtent block_extent(const Geo& g, uint32_t tile) {
  // a head's block grid holds fewer than 2^28 blocks: 32-bit arithmetic
  const uint32_t nyx = (uint32_t)g.ny * (uint32_t)g.nx;
  const uint32_t bt = tile / nyx, rem = tile - bt * nyx;
  const uint32_t by = rem / (uint32_t)g.nx, bx = rem - by * (uint32_t)g.nx;
  BlockExtent e;
  e.lt = min(g.tt, g.T - (int32_t)bt * g.tt);
  e.ly = min(g.th, g.H - (int32_t)by * g.th);
  e.lx = min(g.tw, g.W - (int32_t)bx * g.tw);
  e.full = e.lt == g.tt && e.ly == g.th && e.lx == g.tw;
  return e;
}
// Whether in-block position r exists (block sizes are powers of two).
__device__ __forceinline__ bool pos_exists(const Geo& g, const BlockExtent& e, int r) {
  const int ltw = __builtin_ctz(g.tw), lth = __builtin_ctz(g.th);
  return (r >> (ltw + lth)) < e.lt && ((r >> ltw) & (g.th - 1)) < e.ly && (r & (g.tw - 1)) < e.lx;
}

// First token (within one batch/head) of clip block `tile`: the token of its
// position 0, which always exists.
__device__ __forceinline__ int64_t block_first_token(const Geo& g, uint32_t tile) {
  const uint32_t nyx = (uint32_t)g.ny * (uint32_t)g.nx;
  const uint32_t bt = tile / nyx, rem = tile - bt * nyx;
  const uint32_t by = rem / (uint32_t)g.nx, bx = rem - by * (uint32_t)g.nx;
  return ((int64_t)bt * g.tt * g.H + (int64_t)by * g.th) * g.W + (int64_t)bx * g.tw;
}
// Token offset of in-block position r from the block's first token (block
// sizes are powers of two, so the position is a bit-field code of (t, y, x)).
__device__ __forceinline__ int64_t pos_token_offset(const Geo& g, int r) {
  const int ltw = __builtin_ctz(g.tw), lth = __builtin_ctz(g.th);
  return ((int64_t)(r >> (ltw + lth)) * g.H + ((r >> ltw) & (g.th - 1))) * g.W + (r & (g.tw - 1));
}

// 32-bit forms for the attention kernels, whose per-head offsets fit 32 bits
// (one head's tensor is below 2^31 bytes).  Because the position is a
// bit-field code, positions with disjoint bits add:
// in_block_offset(a + b) = in_block_offset(a) + in_block_offset(b).
__device__ __forceinline__ uint32_t block_origin32(const Geo& g, uint32_t tile) {
  const uint32_t nyx = (uint32_t)g.ny * (uint32_t)g.nx;
  const uint32_t bt = tile / nyx, rem = tile - bt * nyx;
  const uint32_t by = rem / (uint32_t)g.nx, bx = rem - by * (uint32_t)g.nx;
  return ((bt * (uint32_t)g.tt) * (uint32_t)g.H + by * (uint32_t)g.th) * (uint32_t)g.W +
         bx * (uint32_t)g.tw;
}
__device__ __forceinline__ uint32_t in_block_offset(const Geo& g, int r) {
  const int ltw = __builtin_ctz(g.tw), lth = __builtin_ctz(g.th);
  const int it = r >> (ltw + lth), iy = (r >> ltw) & (g.th - 1), ix = r & (g.tw - 1);
  return (uint32_t)((it * g.H + iy) * g.W + ix);
}

hipError_t launch_tile_pool(const Geo& g, const void* x, void* x_tiled, int layout,
                            float* pooled, hipStream_t s);
hipError_t launch_tile_unpermute(const Geo& g, const void* x_tiled, void* x, hipStream_t s);

// Step 2 scoring.  qhat, khat: [bh][n][128] normalised means; red: [bh][n]
// Score_r; part: [bh][red_groups(n)][n] partial sums of Score_r (one per
// group of kRedGroup key blocks).
constexpr int kRedGroup = 128;
int red_groups(int64_t n);
struct ScoreArgs {
  const float* q_pooled;
  const float* k_pooled;
  float* qhat;
  float* khat;
  float* red;
  float* part;
  float lambda_, beta;
};
// normalise both means, then Score_r
hipError_t launch_score_prepare(const Geo& g, const ScoreArgs& a, hipStream_t s);
// the Score_i matrix [bh][n][n] (after launch_score_prepare)
hipError_t launch_score_matrix(const Geo& g, const ScoreArgs& a, float* scores, hipStream_t s);

struct TopkArgs {
  float* scores;        // [bh][n][n] Score_i, written then read by launch_select
  int32_t* topk_idx;
  int32_t k;            // requested top-k
  int32_t width;        // row width of topk_idx
  int32_t exclude_window;
  int32_t wt, wh, ww;
};
// Score_i into t.scores, then the per-row top-k (after launch_score_prepare)
hipError_t launch_select(const Geo& g, const ScoreArgs& a, const TopkArgs& t, hipStream_t s);

struct MaskArgs {
  const int32_t* topk_idx;
  int32_t k_width;
  int32_t* kv_idx;
  int32_t* kv_cnt;
  uint32_t* bitmask;
  int32_t max_kept;
  int32_t wt, wh, ww;
  int32_t combine_and;
};
hipError_t launch_build_mask(const Geo& g, const MaskArgs& a, hipStream_t s);

struct AttnArgs {
  const void* q_t;
  const void* k_t;
  const void* v_t;          // token_io: token-major V; else dim-major tiles
  const int32_t* kv_idx;   // nullptr: dense
  const int32_t* kv_cnt;
  int32_t max_kept;
  void* o_t;
  float* lse;
  float scale_log2;        // softmax scale * log2(e)
  int32_t token_io;        // 1: q_t, k_t, v_t, o_t are token-major [B, h, S, 128]
};
hipError_t launch_attention(const Geo& g, const AttnArgs& a, hipStream_t s);

// Backward of the block-sparse attention (kept lists held fixed).
struct BwdArgs {
  const void* q;          // token-major bf16 [bh][N][128]
  const void* k;
  const void* v;
  const void* dout;
  const float* ld;        // [bh][n][128][2]: (lse * log2(e), D = dO . O) per query
  const int32_t* kv_idx;  // query block -> kept key blocks (NULL: dense)
  const int32_t* kv_cnt;
  int32_t max_kept;
  const int32_t* q_idx;   // key block -> query blocks that keep it, ascending (NULL: dense)
  const int32_t* q_cnt;
  int32_t q_width;
  const int32_t* order;   // per head, key blocks by decreasing q_cnt (NULL: grid order)
  void* dq;               // token-major bf16 outputs
  void* dk;
  void* dv;
  float scale, scale_log2;
};
hipError_t launch_attention_bwd_prep(const Geo& g, const void* o, const void* dout,
                                     const float* lse, float* ld, hipStream_t s);
hipError_t launch_transpose_lists(const Geo& g, const int32_t* kv_idx, const int32_t* kv_cnt,
                                  int32_t max_kept, uint32_t* mask_t, int32_t* q_idx,
                                  int32_t* q_cnt, int32_t* order, hipStream_t s);
hipError_t launch_attention_bwd(const Geo& g, const BwdArgs& a, hipStream_t s);

// Sustained matrix-core rate (measurement aid; see k_calib.hip).
hipError_t launch_calibrate_mfma(const void* operands, float* sink, int grid, int iters,
                                 hipStream_t s);

}  // namespace ssta

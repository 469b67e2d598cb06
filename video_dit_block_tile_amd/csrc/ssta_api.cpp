// Host side of libssta.so: argument validation, device checks and kernel
// dispatch behind the C ABI declared in include/ssta.h.
//
// Every argument is checked before the first HIP call, so a rejected call
// enqueues nothing and the checks can be exercised on a machine without a
// GPU.  The library holds no device memory and no state beyond a per-device
// cache of the architecture check.
#include "ssta.h"

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "ssta_internal.h"

namespace {

using ssta::Geo;

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

bool is_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_ptr(const void* p, bool nullable) {
  if (p == nullptr) return nullable ? SSTA_OK : SSTA_ERR_ARG;
  return is_aligned16(p) ? SSTA_OK : SSTA_ERR_ALIGN;
}

int check_geom(const ssta_geom_t* g, Geo* out) {
  if (g == nullptr) return SSTA_ERR_ARG;
  if (g->batch < 1 || g->heads < 1 || g->head_dim < 1 || g->T < 1 || g->H < 1 || g->W < 1 ||
      g->tile_t < 1 || g->tile_h < 1 || g->tile_w < 1)
    return SSTA_ERR_ARG;
  if (g->text_len < 0) return SSTA_ERR_ARG;
  if (g->head_dim != ssta::kHeadDim) return SSTA_ERR_SHAPE;
  const int64_t R = (int64_t)g->tile_t * g->tile_h * g->tile_w;
  if (R != ssta::kTileTokens && R != ssta::kSmallTile) return SSTA_ERR_SHAPE;
  const int64_t N = (int64_t)g->T * g->H * g->W;
  const int64_t bh = (int64_t)g->batch * g->heads;
  // The block grid rounds up: a grid the block size does not divide has
  // partial blocks on its far edges.
  const int64_t nt = (g->T + g->tile_t - 1) / g->tile_t;
  const int64_t ny = (g->H + g->tile_h - 1) / g->tile_h;
  const int64_t nx = (g->W + g->tile_w - 1) / g->tile_w;
  const int64_t n = nt * ny * nx;
  // A joint sequence appends text_len tokens in blocks of R after the clip's.
  const int64_t n_txt = (g->text_len + R - 1) / R;
  const int64_t S = N + g->text_len, rows = n + n_txt;
  // Every element offset must fit in int64 and every grid in 31 bits.
  if (S > (int64_t(1) << 40) / bh) return SSTA_ERR_SHAPE;
  if (bh * rows > 0x7FFFFFFF) return SSTA_ERR_SHAPE;
  if (rows > 0x7FFFFFFF / 8) return SSTA_ERR_SHAPE;
  out->batch = g->batch;
  out->heads = g->heads;
  out->D = g->head_dim;
  out->T = g->T;
  out->H = g->H;
  out->W = g->W;
  out->tt = g->tile_t;
  out->th = g->tile_h;
  out->tw = g->tile_w;
  out->R = (int32_t)R;
  out->nt = (int32_t)nt;
  out->ny = (int32_t)ny;
  out->nx = (int32_t)nx;
  out->N = N;
  out->n_tiles = n;
  out->bh = bh;
  out->ragged = (g->T % g->tile_t || g->H % g->tile_h || g->W % g->tile_w) ? 1 : 0;
  out->L = g->text_len;
  out->n_txt = (int32_t)n_txt;
  out->S = S;
  out->n_rows = rows;
  return SSTA_OK;
}

int check_params(const ssta_params_t* p) {
  if (p == nullptr) return SSTA_ERR_ARG;
  if (p->win_t < 0 || p->win_h < 0 || p->win_w < 0 || p->topk < 0) return SSTA_ERR_ARG;
  if (!std::isfinite(p->lambda_) || !std::isfinite(p->beta)) return SSTA_ERR_ARG;
  if (!std::isfinite(p->scale) || !(p->scale > 0.0f)) return SSTA_ERR_ARG;
  if (p->flags & ~(SSTA_COMBINE_AND | SSTA_TOPK_EXCLUDE_WINDOW)) return SSTA_ERR_ARG;
  return SSTA_OK;
}

int64_t axis_span(int64_t half, int64_t n) { return half * 2 + 1 < n ? half * 2 + 1 : n; }
int64_t axis_corner(int64_t half, int64_t n) { return half + 1 < n ? half + 1 : n; }

int64_t window_max(const Geo& g, const ssta_params_t* p) {
  return axis_span(p->win_t, g.nt) * axis_span(p->win_h, g.ny) * axis_span(p->win_w, g.nx);
}
int64_t window_min(const Geo& g, const ssta_params_t* p) {
  return axis_corner(p->win_t, g.nt) * axis_corner(p->win_h, g.ny) *
         axis_corner(p->win_w, g.nx);
}

int32_t topk_width(const Geo& g, const ssta_params_t* p) {
  const int64_t cand =
      (p->flags & SSTA_TOPK_EXCLUDE_WINDOW) ? g.n_tiles - window_min(g, p) : g.n_tiles;
  const int64_t w = p->topk < cand ? p->topk : cand;
  return (int32_t)(w > 0 ? w : 0);
}

int32_t max_kept(const Geo& g, const ssta_params_t* p) {
  const int64_t wmax = window_max(g, p), k = topk_width(g, p);
  if (p->flags & SSTA_COMBINE_AND) return (int32_t)(wmax < k ? wmax : k);
  const int64_t u = wmax + k;
  return (int32_t)(u < g.n_tiles ? u : g.n_tiles);
}

constexpr int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

// Scoring workspace: the normalised means, Score_r, its group partials and
// the Score_i matrix the top-k reads.
struct WsLayout {
  int64_t qhat, khat, red, part, scores, total;
};

WsLayout ws_layout(const Geo& g) {
  WsLayout w;
  const int64_t vec = g.bh * g.n_tiles * ssta::kHeadDim * 4;
  w.qhat = 0;
  w.khat = align256(vec);
  w.red = w.khat + align256(vec);
  w.part = w.red + align256(g.bh * g.n_tiles * 4);
  w.scores = w.part + align256(g.bh * ssta::red_groups(g.n_tiles) * g.n_tiles * 4);
  w.total = w.scores + align256(g.bh * g.n_tiles * g.n_tiles * 4);
  return w;
}

// Scratch of ssta_score_select_noalloc: one array per GPU, held until the
// process ends.  Its name is a host-side stand-in; host code uses only the
// device address hipGetSymbolAddress returns for the current device.
constexpr int64_t kNoAllocScratchBytes = int64_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
std::atomic<uint8_t*> g_scratch_ptr[kMaxDevices];

int check_device() {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
    (void)hipGetLastError();
    return SSTA_ERR_NO_DEVICE;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return SSTA_ERR_NO_DEVICE;
  }
  if (dev >= kMaxDevices) return SSTA_ERR_NO_DEVICE;
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return SSTA_ERR_NO_DEVICE;
    }
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? SSTA_OK : SSTA_ERR_ARCH;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return SSTA_OK;
  g_last_hip_error = (int)e;
  return SSTA_ERR_HIP;
}

#define SSTA_TRY(expr)            \
  do {                            \
    const int _rc = (expr);       \
    if (_rc != SSTA_OK) return _rc; \
  } while (0)

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// The current device's address of `scratch`, looked up on the first call on
// that device (with the device current) and kept.
int scratch_ptr(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return SSTA_ERR_NO_DEVICE;
  }
  uint8_t* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    void* addr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || addr == nullptr) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol);
    ptr = static_cast<uint8_t*>(addr);
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return SSTA_OK;
}

int score_common(const ssta_geom_t* g, const ssta_params_t* p, const float* qp,
                 const float* kp, void* ws, size_t ws_bytes, Geo* geo, WsLayout* lay) {
  SSTA_TRY(check_geom(g, geo));
  SSTA_TRY(check_params(p));
  SSTA_TRY(check_ptr(qp, false));
  SSTA_TRY(check_ptr(kp, false));
  if (geo->n_tiles > ssta::kMaxTopkTiles) return SSTA_ERR_SHAPE;
  if (geo->bh > ssta::kMaxScoreHeads) return SSTA_ERR_SHAPE;
  *lay = ws_layout(*geo);
  if (ws == nullptr || (int64_t)ws_bytes < lay->total) return SSTA_ERR_WORKSPACE;
  SSTA_TRY(check_ptr(ws, false));
  return SSTA_OK;
}

}  // namespace

extern "C" {

int ssta_default_params(ssta_params_t* p, int32_t head_dim) {
  if (p == nullptr || head_dim < 1) return SSTA_ERR_ARG;
  p->win_t = p->win_h = p->win_w = 1;
  p->topk = 0;
  // The excerpt's Python scalars 0.9 and 1 - 0.9 scale fp32 tensors, so they
  // act as their fp32 roundings (1 - 0.9 is formed in double first).
  p->lambda_ = 0.9f;
  p->beta = (float)(1.0 - 0.9);
  p->scale = (float)(1.0 / std::sqrt((double)head_dim));
  p->flags = 0u;
  return SSTA_OK;
}

int ssta_tile_pool(const ssta_geom_t* g, const void* x, void* x_tiled, int32_t layout,
                   float* pooled, void* stream) {
  Geo geo;
  SSTA_TRY(check_geom(g, &geo));
  SSTA_TRY(check_ptr(x, false));
  SSTA_TRY(check_ptr(x_tiled, true));
  SSTA_TRY(check_ptr(pooled, true));
  if (x_tiled == nullptr && pooled == nullptr) return SSTA_ERR_ARG;
  if (layout != SSTA_LAYOUT_TOKEN_MAJOR && layout != SSTA_LAYOUT_DIM_MAJOR) return SSTA_ERR_ARG;
  SSTA_TRY(check_device());
  return hip_status(ssta::launch_tile_pool(geo, x, x_tiled, layout, pooled, as_stream(stream)));
}

int ssta_tile_unpermute(const ssta_geom_t* g, const void* x_tiled, void* x, void* stream) {
  Geo geo;
  SSTA_TRY(check_geom(g, &geo));
  SSTA_TRY(check_ptr(x_tiled, false));
  SSTA_TRY(check_ptr(x, false));
  SSTA_TRY(check_device());
  return hip_status(ssta::launch_tile_unpermute(geo, x_tiled, x, as_stream(stream)));
}

int64_t ssta_block_rows(const ssta_geom_t* g) {
  Geo geo;
  SSTA_TRY(check_geom(g, &geo));
  return geo.n_rows;
}

int32_t ssta_topk_width(const ssta_geom_t* g, const ssta_params_t* p) {
  Geo geo;
  SSTA_TRY(check_geom(g, &geo));
  SSTA_TRY(check_params(p));
  return topk_width(geo, p);
}

int32_t ssta_max_kept(const ssta_geom_t* g, const ssta_params_t* p) {
  Geo geo;
  SSTA_TRY(check_geom(g, &geo));
  SSTA_TRY(check_params(p));
  return max_kept(geo, p);
}

int64_t ssta_workspace_bytes(const ssta_geom_t* g, const ssta_params_t* p) {
  Geo geo;
  SSTA_TRY(check_geom(g, &geo));
  SSTA_TRY(check_params(p));
  return ws_layout(geo).total;
}

namespace {
ssta::ScoreArgs score_args(const ssta_params_t* p, const float* q_pooled, const float* k_pooled,
                           uint8_t* ws, const WsLayout& lay) {
  ssta::ScoreArgs sa;
  sa.q_pooled = q_pooled;
  sa.k_pooled = k_pooled;
  sa.qhat = reinterpret_cast<float*>(ws + lay.qhat);
  sa.khat = reinterpret_cast<float*>(ws + lay.khat);
  sa.red = reinterpret_cast<float*>(ws + lay.red);
  sa.part = reinterpret_cast<float*>(ws + lay.part);
  sa.lambda_ = p->lambda_;
  sa.beta = p->beta;
  return sa;
}

int score_select_into(const Geo& geo, const ssta_params_t* p, const float* q_pooled,
                      const float* k_pooled, int32_t* topk_idx, uint8_t* ws, const WsLayout& lay,
                      int32_t width, hipStream_t st) {
  const ssta::ScoreArgs sa = score_args(p, q_pooled, k_pooled, ws, lay);
  SSTA_TRY(hip_status(ssta::launch_score_prepare(geo, sa, st)));
  ssta::TopkArgs ta;
  ta.scores = reinterpret_cast<float*>(ws + lay.scores);
  ta.topk_idx = topk_idx;
  ta.k = p->topk;
  ta.width = width;
  ta.exclude_window = (p->flags & SSTA_TOPK_EXCLUDE_WINDOW) ? 1 : 0;
  ta.wt = p->win_t;
  ta.wh = p->win_h;
  ta.ww = p->win_w;
  return hip_status(ssta::launch_select(geo, sa, ta, st));
}
}  // namespace

int ssta_score_select(const ssta_geom_t* g, const ssta_params_t* p, const float* q_pooled,
                      const float* k_pooled, int32_t* topk_idx, void* workspace,
                      size_t ws_bytes, void* stream) {
  Geo geo;
  WsLayout lay;
  SSTA_TRY(score_common(g, p, q_pooled, k_pooled, workspace, ws_bytes, &geo, &lay));
  const int32_t width = topk_width(geo, p);
  SSTA_TRY(check_ptr(topk_idx, width == 0));
  SSTA_TRY(check_device());
  if (width == 0) return SSTA_OK;   // nothing to select: topk_idx has no columns
  return score_select_into(geo, p, q_pooled, k_pooled, topk_idx,
                           static_cast<uint8_t*>(workspace), lay, width, as_stream(stream));
}

int ssta_score_select_noalloc(const ssta_geom_t* g, const ssta_params_t* p,
                              const float* q_pooled, const float* k_pooled, int32_t* topk_idx,
                              void* stream) {
  Geo geo;
  SSTA_TRY(check_geom(g, &geo));
  SSTA_TRY(check_params(p));
  SSTA_TRY(check_ptr(q_pooled, false));
  SSTA_TRY(check_ptr(k_pooled, false));
  if (geo.n_tiles > ssta::kMaxTopkTiles) return SSTA_ERR_SHAPE;
  if (geo.bh > ssta::kMaxScoreHeads) return SSTA_ERR_SHAPE;
  // heads per pass: as many as the scratch holds; one head must fit
  Geo part = geo;
  part.bh = 1;
  if (ws_layout(part).total > kNoAllocScratchBytes) return SSTA_ERR_SHAPE;
  int64_t hc = kNoAllocScratchBytes / ws_layout(part).total;
  hc = hc < geo.bh ? hc : geo.bh;
  for (;;) {
    part.bh = hc;
    if (hc == 1 || ws_layout(part).total <= kNoAllocScratchBytes) break;
    --hc;
  }
  const int32_t width = topk_width(geo, p);
  SSTA_TRY(check_ptr(topk_idx, width == 0));
  SSTA_TRY(check_device());
  if (width == 0) return SSTA_OK;
  uint8_t* ws = nullptr;
  SSTA_TRY(scratch_ptr(&ws));
  const int64_t n = geo.n_tiles;
  for (int64_t h0 = 0; h0 < geo.bh; h0 += hc) {
    part.bh = geo.bh - h0 < hc ? geo.bh - h0 : hc;
    const WsLayout lay = ws_layout(part);
    SSTA_TRY(score_select_into(part, p, q_pooled + h0 * n * ssta::kHeadDim,
                               k_pooled + h0 * n * ssta::kHeadDim, topk_idx + h0 * n * width, ws,
                               lay, width, as_stream(stream)));
  }
  return SSTA_OK;
}

int ssta_scores(const ssta_geom_t* g, const ssta_params_t* p, const float* q_pooled,
                const float* k_pooled, float* scores, float* red, void* workspace,
                size_t ws_bytes, void* stream) {
  Geo geo;
  WsLayout lay;
  SSTA_TRY(score_common(g, p, q_pooled, k_pooled, workspace, ws_bytes, &geo, &lay));
  SSTA_TRY(check_ptr(scores, false));
  SSTA_TRY(check_ptr(red, true));
  SSTA_TRY(check_device());
  ssta::ScoreArgs sa = score_args(p, q_pooled, k_pooled, static_cast<uint8_t*>(workspace), lay);
  if (red != nullptr) sa.red = red;
  SSTA_TRY(hip_status(ssta::launch_score_prepare(geo, sa, as_stream(stream))));
  return hip_status(ssta::launch_score_matrix(geo, sa, scores, as_stream(stream)));
}

int ssta_build_mask(const ssta_geom_t* g, const ssta_params_t* p, const int32_t* topk_idx,
                    int32_t* kv_idx, int32_t* kv_cnt, uint32_t* bitmask, void* stream) {
  Geo geo;
  SSTA_TRY(check_geom(g, &geo));
  SSTA_TRY(check_params(p));
  const int32_t width = topk_width(geo, p);
  const int32_t mk = max_kept(geo, p);
  SSTA_TRY(check_ptr(topk_idx, width == 0));
  SSTA_TRY(check_ptr(kv_idx, mk == 0));
  SSTA_TRY(check_ptr(kv_cnt, false));
  SSTA_TRY(check_ptr(bitmask, true));
  SSTA_TRY(check_device());
  ssta::MaskArgs ma;
  ma.topk_idx = topk_idx;
  ma.k_width = width;
  ma.kv_idx = kv_idx;
  ma.kv_cnt = kv_cnt;
  ma.bitmask = bitmask;
  ma.max_kept = mk;
  ma.wt = p->win_t;
  ma.wh = p->win_h;
  ma.ww = p->win_w;
  ma.combine_and = (p->flags & SSTA_COMBINE_AND) ? 1 : 0;
  return hip_status(ssta::launch_build_mask(geo, ma, as_stream(stream)));
}

namespace {
int attention_common(const ssta_geom_t* g, const ssta_params_t* p, const void* q, const void* k,
                     const void* v, const int32_t* kv_idx, const int32_t* kv_cnt,
                     int32_t max_kept_, void* o, float* lse, void* stream, int token_io) {
  Geo geo;
  SSTA_TRY(check_geom(g, &geo));
  SSTA_TRY(check_params(p));
  SSTA_TRY(check_ptr(q, false));
  SSTA_TRY(check_ptr(k, false));
  SSTA_TRY(check_ptr(v, false));
  SSTA_TRY(check_ptr(o, false));
  SSTA_TRY(check_ptr(lse, true));
  // One head's K and V (token-major or tiles) are addressed with 32-bit
  // buffer offsets.
  if (geo.n_rows * int64_t(geo.R) * ssta::kHeadDim * 2 > 0x7FFFFFFF)
    return SSTA_ERR_SHAPE;
  const bool dense = kv_cnt == nullptr;
  if (dense) {
    if (kv_idx != nullptr || max_kept_ != 0) return SSTA_ERR_ARG;
  } else {
    if (max_kept_ < 0 || max_kept_ > geo.n_tiles) return SSTA_ERR_ARG;
    SSTA_TRY(check_ptr(kv_cnt, false));
    SSTA_TRY(check_ptr(kv_idx, max_kept_ == 0));
  }
  SSTA_TRY(check_device());
  ssta::AttnArgs aa;
  aa.q_t = q;
  aa.k_t = k;
  aa.v_t = v;   // token-major (token_io) or dim-major tiles
  aa.kv_idx = kv_idx;
  aa.kv_cnt = kv_cnt;
  aa.max_kept = max_kept_;
  aa.o_t = o;
  aa.lse = lse;
  aa.scale_log2 = p->scale * 1.44269504088896340736f;
  aa.token_io = token_io;
  return hip_status(ssta::launch_attention(geo, aa, as_stream(stream)));
}
}  // namespace

int ssta_attention_fwd(const ssta_geom_t* g, const ssta_params_t* p, const void* q_t,
                       const void* k_t, const void* v_t, const int32_t* kv_idx,
                       const int32_t* kv_cnt, int32_t max_kept_, void* o_t, float* lse,
                       void* stream) {
  return attention_common(g, p, q_t, k_t, v_t, kv_idx, kv_cnt, max_kept_, o_t, lse, stream, 0);
}

int ssta_attention_fwd_tokens(const ssta_geom_t* g, const ssta_params_t* p, const void* q,
                              const void* k, const void* v, const int32_t* kv_idx,
                              const int32_t* kv_cnt, int32_t max_kept_, void* o, float* lse,
                              void* stream) {
  return attention_common(g, p, q, k, v, kv_idx, kv_cnt, max_kept_, o, lse, stream, 1);
}

namespace {
struct BwdLayout {
  int64_t ld, mask, q_idx, q_cnt, order, total;
};
BwdLayout bwd_layout(const Geo& g) {
  BwdLayout w;
  // (lse, D) pairs cover every block (text included); the transposed lists
  // cover the clip's key blocks
  const int64_t rows = g.bh * g.n_tiles;
  w.ld = 0;
  w.mask = w.ld + align256(g.bh * g.n_rows * g.R * 8);
  w.q_idx = w.mask + align256(rows * ((g.n_tiles + 31) / 32) * 4);
  w.q_cnt = w.q_idx + align256(rows * g.n_tiles * 4);
  w.order = w.q_cnt + align256(rows * 4);
  w.total = w.order + align256(rows * 4);
  return w;
}
}  // namespace

int64_t ssta_attention_bwd_workspace_bytes(const ssta_geom_t* g) {
  Geo geo;
  SSTA_TRY(check_geom(g, &geo));
  return bwd_layout(geo).total;
}

int ssta_attention_bwd(const ssta_geom_t* g, const ssta_params_t* p, const void* q,
                       const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, const int32_t* kv_idx, const int32_t* kv_cnt,
                       int32_t max_kept_, void* dq, void* dk, void* dv, void* workspace,
                       size_t ws_bytes, void* stream) {
  Geo geo;
  SSTA_TRY(check_geom(g, &geo));
  SSTA_TRY(check_params(p));
  for (const void* ptr : {q, k, v, o, dout, static_cast<const void*>(lse)})
    SSTA_TRY(check_ptr(ptr, false));
  for (void* ptr : {dq, dk, dv}) SSTA_TRY(check_ptr(ptr, false));
  if (geo.n_rows * int64_t(geo.R) * ssta::kHeadDim * 2 > 0x7FFFFFFF)
    return SSTA_ERR_SHAPE;
  const bool dense = kv_cnt == nullptr;
  if (dense) {
    if (kv_idx != nullptr || max_kept_ != 0) return SSTA_ERR_ARG;
  } else {
    if (max_kept_ < 0 || max_kept_ > geo.n_tiles) return SSTA_ERR_ARG;
    SSTA_TRY(check_ptr(kv_cnt, false));
    SSTA_TRY(check_ptr(kv_idx, max_kept_ == 0));
  }
  const BwdLayout lay = bwd_layout(geo);
  if (workspace == nullptr || (int64_t)ws_bytes < lay.total) return SSTA_ERR_WORKSPACE;
  SSTA_TRY(check_ptr(workspace, false));
  SSTA_TRY(check_device());
  hipStream_t st = as_stream(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* ld = reinterpret_cast<float*>(ws + lay.ld);
  SSTA_TRY(hip_status(ssta::launch_attention_bwd_prep(geo, o, dout, lse, ld, st)));
  int32_t* q_idx = reinterpret_cast<int32_t*>(ws + lay.q_idx);
  int32_t* q_cnt = reinterpret_cast<int32_t*>(ws + lay.q_cnt);
  int32_t* order = reinterpret_cast<int32_t*>(ws + lay.order);
  if (!dense)
    SSTA_TRY(hip_status(ssta::launch_transpose_lists(
        geo, kv_idx, kv_cnt, max_kept_, reinterpret_cast<uint32_t*>(ws + lay.mask), q_idx,
        q_cnt, order, st)));
  ssta::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.ld = ld;
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.max_kept = max_kept_;
  a.q_idx = dense ? nullptr : q_idx;
  a.q_cnt = dense ? nullptr : q_cnt;
  a.q_width = (int32_t)geo.n_tiles;
  a.order = dense ? nullptr : order;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.scale = p->scale;
  a.scale_log2 = p->scale * 1.44269504088896340736f;
  return hip_status(ssta::launch_attention_bwd(geo, a, st));
}

int ssta_calibrate_mfma(const void* operands, float* sink, int32_t grid, int32_t iters,
                        void* stream) {
  if (grid <= 0 || iters <= 0 || operands == nullptr || sink == nullptr) return SSTA_ERR_ARG;
  SSTA_TRY(check_ptr(operands, false));
  SSTA_TRY(check_ptr(sink, false));
  SSTA_TRY(check_device());
  return hip_status(ssta::launch_calibrate_mfma(operands, sink, grid, iters, as_stream(stream)));
}

const char* ssta_status_string(int status) {
  switch (status) {
    case SSTA_OK: return "ok";
    case SSTA_ERR_ARG: return "invalid argument";
    case SSTA_ERR_SHAPE: return "unsupported shape";
    case SSTA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SSTA_ERR_NO_DEVICE: return "no usable HIP device";
    case SSTA_ERR_ARCH: return "current device is not gfx950";
    case SSTA_ERR_HIP: return "HIP launch failed";
    case SSTA_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int ssta_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"

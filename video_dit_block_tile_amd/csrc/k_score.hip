// Step 2 of SSTA (selective mask generation): block-level cosine similarity
// Score_s, key-key redundancy Score_r, importance Score_i and the per-query
// top-k ("HunyuanVideo 1.5 Technical Report" summary page, section "SSTA:
// Selective and Sliding Tile Attention", Step 2; the importance_sampling
// excerpt on the "HunyuanVideo-1.5: An 8.3B-Parameter Video Diffusion Model
// Built for Consumer GPUs" page, section "Under the Hood: SSTA and Muon in
// Detail").
//
// The selection is an integer decided by fp32 arithmetic, so every score is
// computed in one fixed order that any implementation can repeat:
//   * dot products are fmaf chains over the channel index 0..127 ascending,
//     starting at 0.0f (register-tiled fp32 VALU products whose inner loop
//     runs over channels in order: no split-K and no matrix cores, whose
//     internal accumulation order is not sequential);
//   * sqrt and division are IEEE correctly rounded;
//   * the redundancy of key block j sums u(i, j) = (khat_i.khat_j + 1) / 2
//     over i != j in two levels: a partial sum from 0 per group of 128 key
//     blocks (ascending i inside the group), then the partials in ascending
//     group order;
//   * nothing is contracted (this file is built with -ffp-contract=off).
// The dot products are bitwise symmetric (fmaf(a, b, c) == fmaf(b, a, c)),
// so the key-key products are evaluated once per pair of 128-block groups
// (the upper triangle of tiles): a tile's column sums give the partials of
// its column group and its row sums those of its row group.  Score_i is
// written once as an [n][n] matrix (128 x 128 tiles) and read back once by
// the per-row top-k, one wave per row.
// Work per (batch, head): n(n+1)/2 * 128 FMAs for the key-key products
// (about half of n^2 * 128) and n^2 * 128 for Score_s; bound by the fp32
// vector ALU, not by HBM.
#include "ssta_internal.h"

#pragma clang fp contract(off)

namespace ssta {
namespace {

// ------------------------------------------------------------------ normalise

// x / |x| with a sequential fmaf sum of squares; a zero vector stays zero.
// Both the query and the key means in one launch: vectors [0, rows) of p0,
// then [0, rows) of p1.  A workgroup takes 64 consecutive vectors: coalesced
// loads into LDS (row stride 129 floats, so the 64 chains read distinct
// banks), one thread per vector for the chain and the square root, then the
// divisions and coalesced stores by all threads.
constexpr int kNV = 64;               // vectors per workgroup
constexpr int kNPad = kHeadDim + 1;   // LDS row stride (floats)
__global__ __launch_bounds__(256) void k_normalize(const float* __restrict__ p0,
                                                   float* __restrict__ o0,
                                                   const float* __restrict__ p1,
                                                   float* __restrict__ o1, int64_t rows) {
  __shared__ float xs[kNV * kNPad];
  __shared__ float nrm[kNV];
  // the two halves are padded to whole workgroups
  const int64_t per = (rows + kNV - 1) / kNV;
  const bool second = blockIdx.x >= per;
  const float* p = second ? p1 : p0;
  float* out = second ? o1 : o0;
  const int64_t v0 = (int64_t)(second ? blockIdx.x - per : blockIdx.x) * kNV;
  const int nv = (int)min((int64_t)kNV, rows - v0);
  const int t = threadIdx.x;
#pragma unroll
  for (int s = 0; s < kNV * kHeadDim / 4 / 256; ++s) {
    const int f = t + 256 * s, r = f / (kHeadDim / 4), c4 = f % (kHeadDim / 4);
    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (r < nv) a = *reinterpret_cast<const float4*>(p + (v0 + r) * kHeadDim + 4 * c4);
    xs[r * kNPad + 4 * c4 + 0] = a.x;
    xs[r * kNPad + 4 * c4 + 1] = a.y;
    xs[r * kNPad + 4 * c4 + 2] = a.z;
    xs[r * kNPad + 4 * c4 + 3] = a.w;
  }
  __syncthreads();
  if (t < kNV) {
    float ss = 0.0f;
    for (int c = 0; c < kHeadDim; ++c) ss = __builtin_fmaf(xs[t * kNPad + c], xs[t * kNPad + c], ss);
    nrm[t] = __builtin_sqrtf(ss);
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < kNV * kHeadDim / 4 / 256; ++s) {
    const int f = t + 256 * s, r = f / (kHeadDim / 4), c4 = f % (kHeadDim / 4);
    if (r >= nv) continue;
    const float d = nrm[r];
    float4 o;
    if (d == 0.0f) {
      o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else {
      o.x = xs[r * kNPad + 4 * c4 + 0] / d;
      o.y = xs[r * kNPad + 4 * c4 + 1] / d;
      o.z = xs[r * kNPad + 4 * c4 + 2] / d;
      o.w = xs[r * kNPad + 4 * c4 + 3] / d;
    }
    *reinterpret_cast<float4*>(out + (v0 + r) * kHeadDim + 4 * c4) = o;
  }
}

// ------------------------------------------------------------------ Score_r

constexpr int kG = kRedGroup;          // key blocks per group (tile edge): 128
constexpr int kDC = 32;                // channels staged per step
constexpr int kPad = kG + 4;           // staging row stride (floats)
constexpr int kUPad = 65;              // u half-tile row stride (floats): conflict-free rows and columns

// Tile t of the upper triangle of the nb x nb tile grid, row-major: (I, J), I <= J.
__device__ __forceinline__ void tri_tile(int t, int nb, int& I, int& J) {
  I = 0;
  while (t >= nb - I) {
    t -= nb - I;
    ++I;
  }
  J = I + t;
}

// Rows [row0, row0 + kG) x channels [d0, d0 + kDC) of a [n][128] matrix into
// LDS transposed, dst[d - d0][row - row0] with row stride kPad (rows past n
// are zero).
__device__ __forceinline__ void stage_t(float* dst, const float* __restrict__ src, int64_t row0,
                                        int64_t n, int d0) {
#pragma unroll
  for (int s = 0; s < kG * kDC / 4 / 256; ++s) {
    const int f = threadIdx.x + 256 * s;
    const int r = f / (kDC / 4), c4 = f % (kDC / 4);
    const int64_t gr = row0 + r;
    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (gr < n) a = *reinterpret_cast<const float4*>(src + gr * kHeadDim + d0 + 4 * c4);
    dst[(4 * c4 + 0) * kPad + r] = a.x;
    dst[(4 * c4 + 1) * kPad + r] = a.y;
    dst[(4 * c4 + 2) * kPad + r] = a.z;
    dst[(4 * c4 + 3) * kPad + r] = a.w;
  }
}

// One tile (I, J) of u(i, j) = (khat_i.khat_j + 1) * 0.5, i in group I, j in
// group J.  Each thread owns 8 rows x 8 columns (columns 4tj..4tj+3 and
// 64+4tj..64+4tj+3, so the 16 column readers of a wave hit distinct banks).
// Outputs the group partials part[bh][g][x] (sum over the 128 key blocks i of
// group g, i != x, ascending i, from +0): the tile's column sums are group
// I's partials of the columns in J; for I != J its row sums are group J's
// partials of the rows in I (u is symmetric).  Every (g, x) is written by
// exactly one tile.  The u tile passes through LDS in two halves of 64
// columns (the row sums carry over from the first half to the second), so
// the workgroup needs only the 34 KB of its staging buffers.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void k_red_tile(const float* __restrict__ khat, float* __restrict__ part, int64_t n, int nb,
                int tiles) {
  __shared__ __attribute__((aligned(16))) float sm[2 * kDC * kPad];   // staging, then u halves
  float* As = sm;
  float* Bs = sm + kDC * kPad;
  const int64_t bh = blockIdx.x / tiles;
  int I, J;
  tri_tile((int)(blockIdx.x % tiles), nb, I, J);
  // The last group may be partial.  Off the diagonal it goes to the row side
  // (I > J), where the waves whose 32 rows all lie past n skip their
  // products: the tile then holds the transpose, and since u is bitwise
  // symmetric, its column and row sums are the same partials.
  if (I < J && (int64_t)(J + 1) * kG > n) {
    const int x = I;
    I = J;
    J = x;
  }
  const int64_t i0 = (int64_t)I * kG, j0 = (int64_t)J * kG;
  const float* kb = khat + bh * n * kHeadDim;
  const int t = threadIdx.x, ti = t >> 4, tj = t & 15;
  const bool live = i0 + 32 * (t >> 6) < n;   // wave-uniform
  float acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.0f;
  for (int dc = 0; dc < kHeadDim; dc += kDC) {
    __syncthreads();   // the previous step's staging is read
    stage_t(As, kb, i0, n, dc);
    stage_t(Bs, kb, j0, n, dc);
    __syncthreads();
    if (!live) continue;
#pragma unroll 4
    for (int d = 0; d < kDC; ++d) {
      const float4 x0 = *reinterpret_cast<const float4*>(&As[d * kPad + 8 * ti]);
      const float4 x1 = *reinterpret_cast<const float4*>(&As[d * kPad + 8 * ti + 4]);
      const float4 y0 = *reinterpret_cast<const float4*>(&Bs[d * kPad + 4 * tj]);
      const float4 y1 = *reinterpret_cast<const float4*>(&Bs[d * kPad + 64 + 4 * tj]);
      const float xa[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      const float yb[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = __builtin_fmaf(xa[a], yb[b], acc[a][b]);
    }
  }
  const int64_t rows = min((int64_t)kG, n - i0), cols = min((int64_t)kG, n - j0);
  float* pb = part + bh * nb * n;
  const int rr = t - kG;   // the row summed by threads kG..2kG-1
  float rsum = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    __syncthreads();   // staging (h = 0) or the previous half (h = 1) is read
    // u[r][c] for the tile-local columns 64h + c, c < 64; the diagonal
    // (i == j) is +0, which leaves a running sum of these non-negative terms
    // bit-identical to skipping it
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        const int r = 8 * ti + a, c = 4 * tj + b4;
        const float u = (acc[a][4 * h + b4] + 1.0f) * 0.5f;
        sm[r * kUPad + c] = (i0 + r == j0 + 64 * h + c) ? 0.0f : u;
      }
    __syncthreads();
    if (t < 64) {
      // column sums: group I's partial of column j0 + 64h + t
      if (64 * h + t < cols) {
        float s = 0.0f;
        for (int r = 0; r < rows; ++r) s = s + sm[r * kUPad + t];
        pb[(int64_t)I * n + j0 + 64 * h + t] = s;
      }
    } else if (t >= kG && I != J && rr < rows) {
      // row sums, columns ascending: group J's partial of row i0 + rr
      const int cend = (int)min((int64_t)64, cols - 64 * h);
      for (int c = 0; c < cend; ++c) rsum = rsum + sm[rr * kUPad + c];
    }
  }
  if (t >= kG && I != J && rr < rows) pb[(int64_t)J * n + i0 + rr] = rsum;
}

// red[bh][x] = (sum over groups g ascending of part[bh][g][x]) / (n - 1).
__global__ __launch_bounds__(256) void k_red_final(const float* __restrict__ part,
                                                   float* __restrict__ red, int64_t n, int nb,
                                                   int64_t total) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t bh = t / n, x = t % n;
  const float* p = part + bh * nb * n + x;
  float s = 0.0f;
  for (int g = 0; g < nb; ++g) s = s + p[(int64_t)g * n];
  red[t] = (n > 1) ? s / (float)(n - 1) : 0.0f;
}

// ------------------------------------------------------------------ Score_i

// Score_i = (lambda * ((qhat_i.khat_j + 1) * 0.5)) - (beta * red_j): two
// rounded products and one rounded difference.
__device__ __forceinline__ float importance(float dot, float red, float lambda_, float beta) {
  const float gs = (dot + 1.0f) * 0.5f;
  const float la = lambda_ * gs;
  const float rb = beta * red;
  return la - rb;
}

// The Score_i matrix [bh][n][n]: 128 x 128 tiles, 8 x 8 per thread, staged
// like the key-key tiles; waves whose 32 query rows all lie past n skip their
// products.
__global__ __launch_bounds__(256) void k_score_matrix(const float* __restrict__ qhat,
                                                       const float* __restrict__ khat,
                                                       const float* __restrict__ red,
                                                       float* __restrict__ scores, int64_t n,
                                                       int64_t tiles1, float lambda_, float beta) {
  __shared__ __attribute__((aligned(16))) float sm[2 * kDC * kPad];
  float* As = sm;
  float* Bs = sm + kDC * kPad;
  const int64_t per = tiles1 * tiles1;
  const int64_t bh = blockIdx.x / per, rem = blockIdx.x % per;
  const int64_t i0 = (rem / tiles1) * kG, j0 = (rem % tiles1) * kG;
  const float* qb = qhat + bh * n * kHeadDim;
  const float* kb = khat + bh * n * kHeadDim;
  const int t = threadIdx.x, ti = t >> 4, tj = t & 15;
  const bool live = i0 + 32 * (t >> 6) < n;   // wave-uniform
  float acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.0f;
  for (int dc = 0; dc < kHeadDim; dc += kDC) {
    __syncthreads();
    stage_t(As, qb, i0, n, dc);
    stage_t(Bs, kb, j0, n, dc);
    __syncthreads();
    if (!live) continue;
#pragma unroll 4
    for (int d = 0; d < kDC; ++d) {
      const float4 x0 = *reinterpret_cast<const float4*>(&As[d * kPad + 8 * ti]);
      const float4 x1 = *reinterpret_cast<const float4*>(&As[d * kPad + 8 * ti + 4]);
      const float4 y0 = *reinterpret_cast<const float4*>(&Bs[d * kPad + 4 * tj]);
      const float4 y1 = *reinterpret_cast<const float4*>(&Bs[d * kPad + 64 + 4 * tj]);
      const float xa[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      const float yb[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = __builtin_fmaf(xa[a], yb[b], acc[a][b]);
    }
  }
  float* sb = scores + bh * n * n;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int64_t j = j0 + (b < 4 ? 4 * tj + b : 64 + 4 * tj + b - 4);
    if (j >= n) continue;
    const float rj = red[bh * n + j];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int64_t i = i0 + 8 * ti + a;
      if (i < n) sb[i * n + j] = importance(acc[a][b], rj, lambda_, beta);
    }
  }
}

// ------------------------------------------------------------------ top-k

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0 is mapped like +0 so that the two compare equal.  Every finite value
// maps above 0, which marks "not a candidate".
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f == 0.0f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Per-row top-k, one wave per query-block row.  Each lane keeps E keys
// (columns lane, lane+64, ...).  The k-th largest key T is found bit by bit
// from the top: thr holds the bits of T found so far and count(key >= thr)
// stays >= want, each step trying the next bit.  Two shortcuts leave T
// unchanged: the bits that all the row's candidate keys share are taken as
// they are, and the search stops at a prefix that exactly want keys reach
// (those are then the row's top want, so the selection below keeps exactly
// them).  Once at most 64 * C2 keys reach thr, those keys (every key that can
// still be selected) are moved with their ids, in ascending id order, into
// C2 slots per lane, and the search and the selection continue on the slots
// alone.  The row keeps every key above T and the lowest-id keys equal to T
// until want are kept, writing ids ascending.
template <int E>
__device__ __forceinline__ int count_ge(const uint32_t (&key)[E], uint32_t c) {
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) cnt += __popcll(__ballot(key[e] >= c));
  return cnt;
}

// Narrow thr from bit `bit` down; returns when done (exactly want keys reach
// thr, or no bit is left) or, when C2 > 0, once count(key >= thr) <= 64 * C2.
template <int E, int C2>
__device__ __forceinline__ bool narrow(const uint32_t (&key)[E], int want, uint32_t& thr,
                                       int& bit, int& reach) {
  for (; bit >= 0; --bit) {
    if (C2 > 0 && reach <= 64 * C2) return false;
    const uint32_t cand = thr | (1u << bit);
    const int cnt = count_ge<E>(key, cand);
    if (cnt >= want) {
      thr = cand;
      reach = cnt;
      if (cnt == want) {
        bit = -1;
        return true;
      }
    }
  }
  return true;
}

// Keep the keys above thr and the lowest-id keys equal to thr until want are
// kept; ids of slot e of lane l are id[e] (ascending in (e, l) order).
template <int E>
__device__ __forceinline__ int select_ids(const uint32_t (&key)[E], const int32_t (&id)[E],
                                          uint32_t thr, int want, int lane, int32_t* o) {
  int above = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) above += __popcll(__ballot(key[e] > thr));
  const int need = want - above;   // >= 1
  int ties = 0, pos = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool eq = key[e] == thr;
    const uint64_t eqm = __ballot(eq);
    const bool sel = key[e] > thr || (eq && ties + lanes_below(eqm) < need);
    ties += __popcll(eqm);
    const uint64_t selm = __ballot(sel);
    if (sel) o[pos + lanes_below(selm)] = id[e];
    pos += __popcll(selm);
  }
  (void)lane;
  return pos;
}

template <int E, int C2>
__global__ __launch_bounds__(256) void k_topk(Geo g, const float* __restrict__ scores,
                                              int32_t* __restrict__ out, int64_t rows, int k,
                                              int width, int excl, int wt, int wh, int ww) {
  constexpr int kSlots = C2 > 0 ? C2 : 1;
  __shared__ uint32_t ckey[4][64 * kSlots];
  __shared__ int32_t cid[4][64 * kSlots];
  const int w = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + w;
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int n = (int)g.n_tiles;                 // at most kMaxTopkTiles (host check)
  const float* s = scores + row * n;
  // All E loads are issued before any is used: a lane past the row's end
  // reads the row's last score (in bounds) and drops it.
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = s[min(lane + 64 * e, n - 1)];
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = lane + 64 * e < n ? order_key(v[e]) : 0u;
  if (excl) {
    // top-k outside the window: blocks inside query block i's window are
    // not candidates
    const int i = (int)(row % n), nyx = g.ny * g.nx;
    const int ti = i / nyx, yi = (i / g.nx) % g.ny, xi = i % g.nx;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = lane + 64 * e;
      const int tj = j / nyx, yj = (j / g.nx) % g.ny, xj = j % g.nx;
      if (abs(tj - ti) <= wt && abs(yj - yi) <= wh && abs(xj - xi) <= ww) key[e] = 0u;
    }
  }
  int ncand = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) ncand += __popcll(__ballot(key[e] != 0u));
  const int want = min(min(k, width), ncand);
  int32_t* o = out + row * width;
  int pos = 0;
  if (want > 0) {
    bool fast = false;
    if (C2 > 0 && want <= 64) {
      // L: the want-th largest of the lanes' largest keys.  want lanes hold a
      // key >= L, so the row's want-th largest key is >= L and every key that
      // can be selected is >= L.  Usually few keys reach L: then they go,
      // ascending ids, to the slots, and the search runs there alone.
      uint32_t lm = 0u;
#pragma unroll
      for (int e = 0; e < E; ++e) lm = max(lm, key[e]);
      uint32_t L = 0u;
      for (int b = 31; b >= 0; --b) {
        const uint32_t cand = L | (1u << b);
        if ((int)__popcll(__ballot(lm >= cand)) >= want) L = cand;
      }
      if (L != 0u) {
        int base = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const bool in = key[e] >= L;
          const uint64_t m = __ballot(in);
          const int at = base + lanes_below(m);
          if (in && at < 64 * kSlots) {
            ckey[w][at] = key[e];
            cid[w][at] = lane + 64 * e;
          }
          base += __popcll(m);
        }
        if (base <= 64 * kSlots) {
          fast = true;
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          uint32_t k2[kSlots];
          int32_t i2[kSlots];
#pragma unroll
          for (int c = 0; c < kSlots; ++c) {
            const int at = 64 * c + lane;
            k2[c] = at < base ? ckey[w][at] : 0u;
            i2[c] = at < base ? cid[w][at] : 0;
          }
          uint32_t kmax = 0u, kmin = ~0u;
#pragma unroll
          for (int c = 0; c < kSlots; ++c)
            if (k2[c] != 0u) {
              kmax = max(kmax, k2[c]);
              kmin = min(kmin, k2[c]);
            }
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
            kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
          }
          const uint32_t diff = kmax ^ kmin;
          int bit = diff ? 31 - __builtin_clz(diff) : -1;
          uint32_t thr = bit < 0 ? kmax : (bit == 31 ? 0u : kmax & ~((2u << bit) - 1u));
          int reach = base;
          narrow<kSlots, 0>(k2, want, thr, bit, reach);
          pos = select_ids<kSlots>(k2, i2, thr, want, lane, o);
        }
      }
    }
    if (!fast) {
      uint32_t kmax = 0u, kmin = ~0u;   // over the candidates (key != 0)
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (key[e] != 0u) {
          kmax = max(kmax, key[e]);
          kmin = min(kmin, key[e]);
        }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
      }
      const uint32_t diff = kmax ^ kmin;
      // top: highest bit in which two candidates differ; the bits above it are
      // common to all candidates, so the search would set exactly those of
      // them that are set in every key (every candidate reaches thr)
      int bit = diff ? 31 - __builtin_clz(diff) : -1;
      uint32_t thr = bit < 0 ? kmax : (bit == 31 ? 0u : kmax & ~((2u << bit) - 1u));
      int reach = ncand;
      const bool done = narrow<E, C2>(key, want, thr, bit, reach);
      if (C2 > 0 && !done) {
        // at most 64 * C2 keys reach thr: move them, ascending ids, to the slots
        int base = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const bool in = key[e] != 0u && key[e] >= thr;
          const uint64_t m = __ballot(in);
          if (in) {
            const int at = base + lanes_below(m);
            ckey[w][at] = key[e];
            cid[w][at] = lane + 64 * e;
          }
          base += __popcll(m);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        uint32_t k2[kSlots];
        int32_t i2[kSlots];
#pragma unroll
        for (int c = 0; c < kSlots; ++c) {
          const int at = 64 * c + lane;
          k2[c] = at < base ? ckey[w][at] : 0u;
          i2[c] = at < base ? cid[w][at] : 0;
        }
        narrow<kSlots, 0>(k2, want, thr, bit, reach);
        pos = select_ids<kSlots>(k2, i2, thr, want, lane, o);
      } else {
        int32_t id[E];
#pragma unroll
        for (int e = 0; e < E; ++e) id[e] = lane + 64 * e;
        pos = select_ids<E>(key, id, thr, want, lane, o);
      }
    }
  }
  for (int p = pos + lane; p < width; p += 64) o[p] = -1;
}

template <int E, int C2>
hipError_t launch_topk_e(const Geo& g, const TopkArgs& a, hipStream_t s) {
  const int64_t rows = g.bh * g.n_tiles;
  hipLaunchKernelGGL((k_topk<E, C2>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, g,
                     a.scores, a.topk_idx, rows, a.k, a.width, a.exclude_window, a.wt, a.wh,
                     a.ww);
  return hipGetLastError();
}

// Slots for the narrowed keys: 2 (up to 128 keys) or 4 (up to 256) per lane;
// none for short rows or a requested k above 192.
template <int E>
hipError_t launch_topk_c(const Geo& g, const TopkArgs& a, hipStream_t s) {
  const int kw = min(a.k, a.width);
  if (E >= 4 && kw <= 64) return launch_topk_e<E, 2>(g, a, s);
  if (E >= 8 && kw <= 192) return launch_topk_e<E, 4>(g, a, s);
  return launch_topk_e<E, 0>(g, a, s);
}

}  // namespace

int red_groups(int64_t n) { return (int)((n + kRedGroup - 1) / kRedGroup); }

hipError_t launch_score_prepare(const Geo& g, const ScoreArgs& a, hipStream_t s) {
  const int64_t n = g.n_tiles;
  const int64_t vecs = g.bh * n;
  hipLaunchKernelGGL(k_normalize, dim3((unsigned)(2 * ((vecs + kNV - 1) / kNV))), dim3(256), 0,
                     s, a.q_pooled, a.qhat, a.k_pooled, a.khat, vecs);
  const int nb = red_groups(n);
  const int tiles = nb * (nb + 1) / 2;
  hipLaunchKernelGGL(k_red_tile, dim3((unsigned)(g.bh * tiles)), dim3(256), 0, s, a.khat, a.part,
                     n, nb, tiles);
  hipLaunchKernelGGL(k_red_final, dim3((unsigned)((vecs + 255) / 256)), dim3(256), 0, s, a.part,
                     a.red, n, nb, vecs);
  return hipGetLastError();
}

hipError_t launch_score_matrix(const Geo& g, const ScoreArgs& a, float* scores, hipStream_t s) {
  const int64_t t1 = (g.n_tiles + kG - 1) / kG;
  hipLaunchKernelGGL(k_score_matrix, dim3((unsigned)(g.bh * t1 * t1)), dim3(256), 0, s, a.qhat,
                     a.khat, a.red, scores, g.n_tiles, t1, a.lambda_, a.beta);
  return hipGetLastError();
}

hipError_t launch_select(const Geo& g, const ScoreArgs& a, const TopkArgs& t, hipStream_t s) {
  const hipError_t e = launch_score_matrix(g, a, t.scores, s);
  if (e != hipSuccess) return e;
  const int64_t slots = (g.n_tiles + 63) / 64;   // keys per lane
  if (slots <= 1) return launch_topk_c<1>(g, t, s);
  if (slots <= 2) return launch_topk_c<2>(g, t, s);
  if (slots <= 4) return launch_topk_c<4>(g, t, s);
  if (slots <= 8) return launch_topk_c<8>(g, t, s);
  if (slots <= 16) return launch_topk_c<16>(g, t, s);
  if (slots <= 32) return launch_topk_c<32>(g, t, s);
  return launch_topk_c<64>(g, t, s);
}

}  // namespace ssta

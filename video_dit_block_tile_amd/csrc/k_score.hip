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
//     starting at 0.0f (an LDS-tiled fp32 VALU GEMM whose inner loop runs
//     over channels in order: no split-K, no matrix cores, whose internal
//     accumulation order is not sequential; channels are staged in two LDS
//     chunks, and each chain simply continues into the second);
//   * sqrt and division are IEEE correctly rounded;
//   * the redundancy sum runs over key blocks in ascending order;
//   * nothing is contracted (this file is built with -ffp-contract=off).
// Work: 2 * n^2 * 128 FMAs per (batch, head) for Q.K and K.K; the kernels are
// bound by the fp32 vector ALU, not by HBM.
#include "ssta_internal.h"

#pragma clang fp contract(off)

namespace ssta {
namespace {

// GEMM tiles: 128 rows x 64 columns per workgroup of 256 threads, each
// thread an 8 x 4 block of dot products; channels staged through LDS in two
// chunks of 64 (each dot product stays one fmaf chain over channels 0..127).
constexpr int kTI = 128;   // rows (query blocks, or key blocks i for Score_r)
constexpr int kTJ = 64;    // columns (key blocks j)
constexpr int kDC = 64;    // channels per LDS chunk

// One thread per vector: x / |x| with a sequential fmaf sum of squares.
__global__ __launch_bounds__(256) void k_normalize(const float* __restrict__ p,
                                                   float* __restrict__ out, int64_t rows) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows) return;
  const float4* v = reinterpret_cast<const float4*>(p + i * kHeadDim);
  float ss = 0.0f;
#pragma unroll 8
  for (int c = 0; c < kHeadDim / 4; ++c) {
    const float4 a = v[c];
    ss = __builtin_fmaf(a.x, a.x, ss);
    ss = __builtin_fmaf(a.y, a.y, ss);
    ss = __builtin_fmaf(a.z, a.z, ss);
    ss = __builtin_fmaf(a.w, a.w, ss);
  }
  const float nrm = __builtin_sqrtf(ss);
  float4* o = reinterpret_cast<float4*>(out + i * kHeadDim);
#pragma unroll 8
  for (int c = 0; c < kHeadDim / 4; ++c) {
    const float4 a = v[c];
    float4 r;
    if (nrm == 0.0f) {
      r = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else {
      r.x = a.x / nrm;
      r.y = a.y / nrm;
      r.z = a.z / nrm;
      r.w = a.w / nrm;
    }
    o[c] = r;
  }
}

// Loads rows [row0, row0+ROWS) x channels [d0, d0+kDC) of a [n][128] fp32
// matrix into LDS transposed, dst[d - d0][row - row0] (rows past n are zero).
template <int ROWS>
__device__ __forceinline__ void load_chunk_t(float (*dst)[ROWS], const float* __restrict__ src,
                                             int64_t row0, int64_t n, int d0) {
#pragma unroll
  for (int it = 0; it < ROWS / 16; ++it) {
    const int q = threadIdx.x + 256 * it;
    const int r = q % ROWS, c4 = q / ROWS;          // 16 chunks of 4 channels
    const int64_t gr = row0 + r;
    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (gr < n) a = *reinterpret_cast<const float4*>(src + gr * kHeadDim + d0 + 4 * c4);
    dst[4 * c4 + 0][r] = a.x;
    dst[4 * c4 + 1][r] = a.y;
    dst[4 * c4 + 2][r] = a.z;
    dst[4 * c4 + 3][r] = a.w;
  }
}

// acc[a][b] = fmaf(A[d][8*ti+a], B[d][4*tj+b], acc[a][b]) for d = 0 .. kDC-1
// in order: continues each chain over one channel chunk.
__device__ __forceinline__ void dots_8x4(const float (*A)[kTI], const float (*B)[kTJ], int ti,
                                         int tj, float acc[8][4]) {
#pragma unroll 4
  for (int d = 0; d < kDC; ++d) {
    const float4 x0 = *reinterpret_cast<const float4*>(&A[d][8 * ti]);
    const float4 x1 = *reinterpret_cast<const float4*>(&A[d][8 * ti + 4]);
    const float4 y = *reinterpret_cast<const float4*>(&B[d][4 * tj]);
    const float xa[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const float yb[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fmaf(xa[a], yb[b], acc[a][b]);
  }
}

// Score_r: one workgroup owns 64 key columns j and walks the key blocks i in
// ascending order, 128 at a time, adding u(i, j) = (khat_i.khat_j + 1) * 0.5
// for i != j into one running fp32 sum per column.
__global__ __launch_bounds__(256) void k_redundancy(const float* __restrict__ khat,
                                                    float* __restrict__ red, int64_t n) {
  __shared__ __attribute__((aligned(16))) float kj[kHeadDim][kTJ];   // the 64 columns
  __shared__ __attribute__((aligned(16))) float ki[kDC][kTI];        // rows; reused for u
  const int64_t bh = blockIdx.y;
  const int64_t j0 = (int64_t)blockIdx.x * kTJ;
  const float* kb = khat + bh * n * kHeadDim;
  const int t = threadIdx.x;
  const int ti = t >> 4, tj = t & 15;
  load_chunk_t<kTJ>(kj, kb, j0, n, 0);
  load_chunk_t<kTJ>(kj + kDC, kb, j0, n, kDC);
  float s = 0.0f;                                   // running sum of column j0 + t (t < 64)
  float (*u)[kTJ] = reinterpret_cast<float (*)[kTJ]>(&ki[0][0]);   // [kTI][kTJ]
  for (int64_t i0 = 0; i0 < n; i0 += kTI) {
    float acc[8][4];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
    for (int dc = 0; dc < kHeadDim; dc += kDC) {
      __syncthreads();                              // ki (or u) free
      load_chunk_t<kTI>(ki, kb, i0, n, dc);
      __syncthreads();
      dots_8x4(ki, kj + dc, ti, tj, acc);
    }
    __syncthreads();                                // everyone done reading ki
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) u[8 * ti + a][4 * tj + b] = (acc[a][b] + 1.0f) * 0.5f;
    __syncthreads();
    // Every u is >= +0 and s starts at +0, so adding +0 in place of the
    // skipped diagonal term leaves s bit-identical; the branch-free form lets
    // the LDS reads run ahead of the dependent adds.
    if (t < kTJ) {
      const int64_t j = j0 + t;
      if (n - i0 >= kTI) {
#pragma unroll 16
        for (int r = 0; r < kTI; ++r) {
          const float v = u[r][t];
          s = s + (i0 + r != j ? v : 0.0f);
        }
      } else {
        const int lim = (int)(n - i0);
        for (int r = 0; r < lim; ++r) {
          const float v = u[r][t];
          s = s + (i0 + r != j ? v : 0.0f);
        }
      }
    }
  }
  if (t < kTJ && j0 + t < n) red[bh * n + j0 + t] = (n > 1) ? s / (float)(n - 1) : 0.0f;
}

// Score_i = (lambda * (qhat_i.khat_j + 1) * 0.5) - (beta * red_j), one
// 128 x 64 tile per workgroup.
__global__ __launch_bounds__(256) void k_score_matrix(const float* __restrict__ qhat,
                                                      const float* __restrict__ khat,
                                                      const float* __restrict__ red,
                                                      float* __restrict__ scores, int64_t n,
                                                      float lambda_, float beta) {
  __shared__ __attribute__((aligned(16))) float qi[kDC][kTI];
  __shared__ __attribute__((aligned(16))) float kj[kDC][kTJ];
  const int64_t bh = blockIdx.z;
  const int64_t i0 = (int64_t)blockIdx.y * kTI, j0 = (int64_t)blockIdx.x * kTJ;
  const int t = threadIdx.x;
  const int ti = t >> 4, tj = t & 15;
  float acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
  for (int dc = 0; dc < kHeadDim; dc += kDC) {
    __syncthreads();
    load_chunk_t<kTI>(qi, qhat + bh * n * kHeadDim, i0, n, dc);
    load_chunk_t<kTJ>(kj, khat + bh * n * kHeadDim, j0, n, dc);
    __syncthreads();
    dots_8x4(qi, kj, ti, tj, acc);
  }
  float* sb = scores + bh * n * n;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int64_t j = j0 + 4 * tj + b;
    if (j >= n) continue;
    const float rb = beta * red[bh * n + j];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int64_t i = i0 + 8 * ti + a;
      if (i >= n) continue;
      const float gs = (acc[a][b] + 1.0f) * 0.5f;
      const float la = lambda_ * gs;
      sb[i * n + j] = la - rb;
    }
  }
}

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
// from the top (one wave-wide count per bit), then the row keeps every key
// above T and the lowest-id columns equal to T until k are kept, writing ids
// ascending.  Two shortcuts leave T's role unchanged: the bits that all the
// row's candidate keys share are taken as they are, and the search stops at
// a prefix that exactly k keys reach (those k are then the row's top k, so
// the selection below keeps exactly them).
template <int E>
__global__ __launch_bounds__(256) void k_topk(Geo g, const float* __restrict__ scores,
                                              int32_t* __restrict__ out, int64_t rows, int k,
                                              int width, int excl, int wt, int wh, int ww) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
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
    // common to all candidates, so the search would set exactly those of them
    // that are set in every key
    const int top = diff ? 31 - __builtin_clz(diff) : -1;
    uint32_t thr = top < 0 ? kmax : (top == 31 ? 0u : kmax & ~((2u << top) - 1u));
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) cnt += __popcll(__ballot(key[e] >= cand));
      if (cnt >= want) {
        thr = cand;
        if (cnt == want) break;
      }
    }
    int above = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) above += __popcll(__ballot(key[e] > thr));
    const int need = want - above;   // >= 1
    int ties = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool eq = key[e] == thr;
      const uint64_t eqm = __ballot(eq);
      const bool sel = key[e] > thr || (eq && ties + lanes_below(eqm) < need);
      ties += __popcll(eqm);
      const uint64_t selm = __ballot(sel);
      if (sel) o[pos + lanes_below(selm)] = (int32_t)(lane + 64 * e);
      pos += __popcll(selm);
    }
  }
  for (int p = pos + lane; p < width; p += 64) o[p] = -1;
}

template <int E>
hipError_t launch_topk_e(const Geo& g, const TopkArgs& a, hipStream_t s) {
  const int64_t rows = g.bh * g.n_tiles;
  hipLaunchKernelGGL(k_topk<E>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, g, a.scores,
                     a.topk_idx, rows, a.k, a.width, a.exclude_window, a.wt, a.wh, a.ww);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scores(const Geo& g, const ScoreArgs& a, hipStream_t s) {
  const int64_t n = g.n_tiles;
  const int64_t vecs = g.bh * n;
  const unsigned nb = (unsigned)((vecs + 255) / 256);
  hipLaunchKernelGGL(k_normalize, dim3(nb), dim3(256), 0, s, a.q_pooled, a.qhat, vecs);
  hipLaunchKernelGGL(k_normalize, dim3(nb), dim3(256), 0, s, a.k_pooled, a.khat, vecs);
  const unsigned cols = (unsigned)((n + kTJ - 1) / kTJ), rows = (unsigned)((n + kTI - 1) / kTI);
  hipLaunchKernelGGL(k_redundancy, dim3(cols, (unsigned)g.bh), dim3(256), 0, s, a.khat, a.red,
                     n);
  hipLaunchKernelGGL(k_score_matrix, dim3(cols, rows, (unsigned)g.bh), dim3(256), 0, s, a.qhat,
                     a.khat, a.red, a.scores, n, a.lambda_, a.beta);
  return hipGetLastError();
}

hipError_t launch_topk(const Geo& g, const TopkArgs& a, hipStream_t s) {
  const int64_t slots = (g.n_tiles + 63) / 64;
  if (slots <= 1) return launch_topk_e<1>(g, a, s);
  if (slots <= 2) return launch_topk_e<2>(g, a, s);
  if (slots <= 4) return launch_topk_e<4>(g, a, s);
  if (slots <= 8) return launch_topk_e<8>(g, a, s);
  if (slots <= 16) return launch_topk_e<16>(g, a, s);
  if (slots <= 32) return launch_topk_e<32>(g, a, s);
  return launch_topk_e<64>(g, a, s);
}

}  // namespace ssta

// Step 1 (3D block partition) and the block means of Step 2 of SSTA
// ("HunyuanVideo 1.5 Technical Report" summary page, section "SSTA: Selective
// and Sliding Tile Attention").
//
// k_tile_pool: one workgroup per (batch*head, block).  The block's 128 tokens
// arrive as runs of tile_w consecutive tokens (one 256-byte row each); every
// thread moves eight 16-byte chunks, so each wave reads whole rows and the
// token-major output is written as one contiguous 32 KB stretch.  The block
// is staged in LDS once for the two consumers that need it column-wise: the
// fp32 mean (a sequential sum per channel, ascending token order) and the
// dim-major copy used for V.
//
// HBM traffic per 128-token block and tensor: 32 KB read + 32 KB written
// (+512 B of means); the kernel is bound by HBM bandwidth.  Blocks of 64
// tokens (e.g. 4x4x4) use the same kernel with half the rows per workgroup.  Edge blocks of a ragged grid
// (a grid the block size does not divide) read only the tokens that exist.
// On a joint video + text sequence the text follows the clip's tokens; tiled
// copies append its 128-token blocks after the clip's, and only clip blocks
// are pooled (the text is kept out of scoring).
#include "ssta_internal.h"

#pragma clang fp contract(off)

namespace ssta {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// One workgroup per (batch*head, block) over `rows` blocks per head: the clip's
// n_tiles, then (when a tiled copy is written) the text blocks of a joint
// sequence.  kR = tokens per block (128 or 64).
template <int kR>
__global__ __launch_bounds__(256) void k_tile_pool(Geo g, const uint16_t* __restrict__ x,
                                                   uint16_t* __restrict__ xt, int layout,
                                                   float* __restrict__ pooled, int64_t rows) {
  constexpr int kM = kR / 16;                     // 16-byte chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t lds[kR * kHeadDim];  // [r][d]
  const int64_t blk = blockIdx.x;                 // bh * rows + tile
  const int64_t bh = blk / rows, tile = blk % rows;
  const int t = threadIdx.x;
  const int ch = t & 15;                          // 16-byte chunk = 8 channels
  const uint16_t* xb = x + bh * g.S * kHeadDim;
  // An edge block of a ragged grid, or the last text block, lacks some
  // positions: they read as zero and do not enter the mean.
  const bool text = tile >= g.n_tiles;
  const int64_t u0 = (tile - g.n_tiles) * kR;   // text: first text token
  const BlockExtent ext = block_extent(g, text ? 0u : (uint32_t)tile);
  const int64_t first = text ? g.N + u0 : block_first_token(g, (uint32_t)tile);

  u32x4 v[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    const int r = (t >> 4) + 16 * m;
    const bool ok = text ? u0 + r < g.L : (ext.full || pos_exists(g, ext, r));
    // a missing position reads the block's first token (which exists), then zero
    const int64_t tok = first + (!ok ? 0 : text ? r : pos_token_offset(g, r));
    v[m] = *reinterpret_cast<const u32x4*>(xb + tok * kHeadDim + ch * 8);
    if (!ok) v[m] = u32x4{0u, 0u, 0u, 0u};
  }
  if (xt != nullptr && layout == 0) {
    uint16_t* ob = xt + blk * (int64_t)(kR * kHeadDim);
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      const int r = (t >> 4) + 16 * m;
      *reinterpret_cast<u32x4*>(ob + r * kHeadDim + ch * 8) = v[m];
    }
  }
  const bool pool_here = pooled != nullptr && !text;   // text blocks have no mean
  const bool need_lds = pool_here || (xt != nullptr && layout == 1);
  if (!need_lds) return;
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    const int r = (t >> 4) + 16 * m;
    *reinterpret_cast<u32x4*>(lds + r * kHeadDim + ch * 8) = v[m];
  }
  __syncthreads();
  if (pool_here && t < kHeadDim) {
    // missing positions hold +0 in LDS, which leaves the running sum exact
    float s = 0.0f;
#pragma unroll 16
    for (int r = 0; r < kR; ++r) s = s + bf16_bits_to_f32(lds[r * kHeadDim + t]);
    const int count = ext.full ? kR : ext.lt * ext.ly * ext.lx;
    pooled[(bh * g.n_tiles + tile) * kHeadDim + t] = s / (float)count;
  }
  if (xt != nullptr && layout == 1) {
    // dim-major: thread owns channel d and kR/2 consecutive tokens
    const int d = t & 127;
    const int r0 = (t >> 7) * (kR / 2);
    uint16_t* ob = xt + blk * (int64_t)(kR * kHeadDim) + d * kR + r0;
#pragma unroll
    for (int q = 0; q < kR / 16; ++q) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = lds[(r0 + 8 * q + 2 * e) * kHeadDim + d];
        const uint32_t hi = lds[(r0 + 8 * q + 2 * e + 1) * kHeadDim + d];
        w[e] = lo | (hi << 16);
      }
      *reinterpret_cast<u32x4*>(ob + 8 * q) = w;
    }
  }
}

template <int kR>
__global__ __launch_bounds__(256) void k_tile_unpermute(Geo g, const uint16_t* __restrict__ xt,
                                                        uint16_t* __restrict__ x) {
  constexpr int kM = kR / 16;
  const int64_t blk = blockIdx.x;                 // bh * n_rows + block
  const int64_t bh = blk / g.n_rows, tile = blk % g.n_rows;
  const int t = threadIdx.x;
  const int ch = t & 15;
  const uint16_t* ib = xt + blk * (int64_t)(kR * kHeadDim);
  uint16_t* ob = x + bh * g.S * kHeadDim;
  const bool text = tile >= g.n_tiles;
  const int64_t u0 = (tile - g.n_tiles) * kR;
  const BlockExtent ext = block_extent(g, text ? 0u : (uint32_t)tile);
  const int64_t first = text ? g.N + u0 : block_first_token(g, (uint32_t)tile);
  u32x4 v[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    const int r = (t >> 4) + 16 * m;
    v[m] = *reinterpret_cast<const u32x4*>(ib + r * kHeadDim + ch * 8);
  }
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    const int r = (t >> 4) + 16 * m;
    if (text ? u0 + r < g.L : (ext.full || pos_exists(g, ext, r)))
      *reinterpret_cast<u32x4*>(ob + (first + (text ? r : pos_token_offset(g, r))) * kHeadDim +
                                ch * 8) = v[m];
  }
}

}  // namespace

hipError_t launch_tile_pool(const Geo& g, const void* x, void* x_tiled, int layout,
                            float* pooled, hipStream_t s) {
  // text blocks are copied, never pooled
  const int64_t rows = x_tiled != nullptr ? g.n_rows : g.n_tiles;
  const int64_t blocks = g.bh * rows;
  if (g.R == kSmallTile)
    hipLaunchKernelGGL(k_tile_pool<kSmallTile>, dim3((unsigned)blocks), dim3(256), 0, s, g,
                       static_cast<const uint16_t*>(x), static_cast<uint16_t*>(x_tiled), layout,
                       pooled, rows);
  else
    hipLaunchKernelGGL(k_tile_pool<kTileTokens>, dim3((unsigned)blocks), dim3(256), 0, s, g,
                       static_cast<const uint16_t*>(x), static_cast<uint16_t*>(x_tiled), layout,
                       pooled, rows);
  return hipGetLastError();
}

hipError_t launch_tile_unpermute(const Geo& g, const void* x_tiled, void* x, hipStream_t s) {
  const int64_t blocks = g.bh * g.n_rows;
  if (g.R == kSmallTile)
    hipLaunchKernelGGL(k_tile_unpermute<kSmallTile>, dim3((unsigned)blocks), dim3(256), 0, s, g,
                       static_cast<const uint16_t*>(x_tiled), static_cast<uint16_t*>(x));
  else
    hipLaunchKernelGGL(k_tile_unpermute<kTileTokens>, dim3((unsigned)blocks), dim3(256), 0, s, g,
                       static_cast<const uint16_t*>(x_tiled), static_cast<uint16_t*>(x));
  return hipGetLastError();
}

}  // namespace ssta

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
// HBM traffic per block and tensor: 32 KB read + 32 KB written (+512 B of
// means); the kernel is bound by HBM bandwidth.  Edge blocks of a ragged grid
// (a grid the block size does not divide) read only the tokens that exist.
#include "ssta_internal.h"

#pragma clang fp contract(off)

namespace ssta {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

__global__ __launch_bounds__(256) void k_tile_pool(Geo g, const uint16_t* __restrict__ x,
                                                   uint16_t* __restrict__ xt, int layout,
                                                   float* __restrict__ pooled) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kTileTokens * kHeadDim];  // [r][d]
  const int64_t blk = blockIdx.x;                 // bh * n_tiles + tile
  const int64_t bh = blk / g.n_tiles, tile = blk % g.n_tiles;
  const int t = threadIdx.x;
  const int ch = t & 15;                          // 16-byte chunk = 8 channels
  const uint16_t* xb = x + bh * g.N * kHeadDim;
  // An edge block of a ragged grid lacks some positions: they read as zero
  // and do not enter the mean.
  const BlockExtent ext = block_extent(g, tile);

  u32x4 v[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int r = (t >> 4) + 16 * m;
    const bool ok = ext.full || pos_exists(g, ext, r);
    const int64_t tok = ok ? tile_token(g, tile, r) : 0;   // a real row either way
    v[m] = *reinterpret_cast<const u32x4*>(xb + tok * kHeadDim + ch * 8);
    if (!ok) v[m] = u32x4{0u, 0u, 0u, 0u};
  }
  if (xt != nullptr && layout == 0) {
    uint16_t* ob = xt + blk * (int64_t)(kTileTokens * kHeadDim);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int r = (t >> 4) + 16 * m;
      *reinterpret_cast<u32x4*>(ob + r * kHeadDim + ch * 8) = v[m];
    }
  }
  const bool need_lds = pooled != nullptr || (xt != nullptr && layout == 1);
  if (!need_lds) return;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int r = (t >> 4) + 16 * m;
    *reinterpret_cast<u32x4*>(lds + r * kHeadDim + ch * 8) = v[m];
  }
  __syncthreads();
  if (pooled != nullptr && t < kHeadDim) {
    // missing positions hold +0 in LDS, which leaves the running sum exact
    float s = 0.0f;
#pragma unroll 16
    for (int r = 0; r < kTileTokens; ++r) s = s + bf16_bits_to_f32(lds[r * kHeadDim + t]);
    const int count = ext.full ? kTileTokens : ext.lt * ext.ly * ext.lx;
    pooled[blk * kHeadDim + t] = s / (float)count;
  }
  if (xt != nullptr && layout == 1) {
    // dim-major: thread owns channel d and 64 consecutive tokens
    const int d = t & 127;
    const int r0 = (t >> 7) * 64;
    uint16_t* ob = xt + blk * (int64_t)(kTileTokens * kHeadDim) + d * kTileTokens + r0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
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

__global__ __launch_bounds__(256) void k_tile_unpermute(Geo g, const uint16_t* __restrict__ xt,
                                                        uint16_t* __restrict__ x) {
  const int64_t blk = blockIdx.x;
  const int64_t bh = blk / g.n_tiles, tile = blk % g.n_tiles;
  const int t = threadIdx.x;
  const int ch = t & 15;
  const uint16_t* ib = xt + blk * (int64_t)(kTileTokens * kHeadDim);
  uint16_t* ob = x + bh * g.N * kHeadDim;
  const BlockExtent ext = block_extent(g, tile);
  u32x4 v[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int r = (t >> 4) + 16 * m;
    v[m] = *reinterpret_cast<const u32x4*>(ib + r * kHeadDim + ch * 8);
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int r = (t >> 4) + 16 * m;
    if (ext.full || pos_exists(g, ext, r))
      *reinterpret_cast<u32x4*>(ob + tile_token(g, tile, r) * kHeadDim + ch * 8) = v[m];
  }
}

}  // namespace

hipError_t launch_tile_pool(const Geo& g, const void* x, void* x_tiled, int layout,
                            float* pooled, hipStream_t s) {
  const int64_t blocks = g.bh * g.n_tiles;
  hipLaunchKernelGGL(k_tile_pool, dim3((unsigned)blocks), dim3(256), 0, s, g,
                     static_cast<const uint16_t*>(x), static_cast<uint16_t*>(x_tiled), layout,
                     pooled);
  return hipGetLastError();
}

hipError_t launch_tile_unpermute(const Geo& g, const void* x_tiled, void* x, hipStream_t s) {
  const int64_t blocks = g.bh * g.n_tiles;
  hipLaunchKernelGGL(k_tile_unpermute, dim3((unsigned)blocks), dim3(256), 0, s, g,
                     static_cast<const uint16_t*>(x_tiled), static_cast<uint16_t*>(x));
  return hipGetLastError();
}

}  // namespace ssta

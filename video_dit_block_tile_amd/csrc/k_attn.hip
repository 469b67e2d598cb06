// Step 4 of SSTA: block-sparse attention over the kept (query block, key
// block) pairs ("HunyuanVideo 1.5 Technical Report" summary page, section
// "SSTA: Selective and Sliding Tile Attention", Step 4 and the attention
// equation): for each query token, softmax of scale*q.k over the tokens of
// the kept key blocks only, then the weighted sum of their values.
//
// gfx950 design.  One workgroup (4 waves) per query block of 128 tokens;
// each wave owns 32 queries.  The kernel computes the transposed scores
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = the
// wave's Q^T held in registers for the whole row), so each lane ends up with
// one query's scores for 64 of the 128 keys of a block and the row softmax
// needs a single cross-lane exchange (lane ^ 32).  The softmax runs online in
// fp32 in the log2 domain.  The probabilities never leave registers: the
// MFMA output layout of S^T is reused directly as the B operand of
// O^T += V^T P^T, with the contraction's key order permuted to match, and V
// arrives dim-major so the A operand (V^T rows) is two 8-byte LDS reads.
// K and V^T tiles (32 KB each) are staged in LDS with a 16-byte-chunk XOR
// swizzle (chunk ^ row%16) so the MFMA operand reads are conflict-free.
// Workgroup ids are remapped so each XCD walks a contiguous range of query
// blocks of one head: neighbouring query blocks share most window blocks,
// which then hit in that XCD's L2.
//
// Work per kept pair: 4*128^3 = 8.39 MFLOP on the matrix cores, 64 KB of
// K/V^T reads.  Bound: bf16 MFMA throughput (and the fp32 softmax that must
// overlap it).
#include "ssta_internal.h"

namespace ssta {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileBytes = kTileTokens * kHeadDim * 2;   // 32 KB

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 256 + ((chunk ^ (row & 15)) << 4);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void k_attn_fwd(Geo g, AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kTileBytes];
  uint8_t* sK = smem;                 // [key][256 B]
  uint8_t* sV = smem + kTileBytes;    // [d][256 B]

  const int64_t nrows = g.bh * g.n_tiles;
  const int64_t row = xcd_remap(blockIdx.x, nrows);
  const int64_t bh = row / g.n_tiles;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  constexpr int64_t kTileElems = kTileTokens * kHeadDim;

  const uint16_t* qb = static_cast<const uint16_t*>(a.q_t) + row * kTileElems;
  const uint8_t* kb = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(a.k_t) +
                                                       bh * g.n_tiles * kTileElems);
  const uint8_t* vb = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(a.v_t) +
                                                       bh * g.n_tiles * kTileElems);
  const bool dense = a.kv_cnt == nullptr;
  const int cnt = dense ? (int)g.n_tiles : a.kv_cnt[row];
  const int32_t* idx = dense ? nullptr : a.kv_idx + row * a.max_kept;

  // B operand of S^T = K Q^T: query (32*wave + l32), channels 16*s + 8*hl .. +8.
  const int qrow = wave * 32 + l32;
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = *reinterpret_cast<const bf16x8*>(qb + qrow * kHeadDim + 16 * s + 8 * hl);

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m = -INFINITY;   // running max of the log2-scaled scores
  float l = 0.0f;        // this lane's part of the running denominator
  const float c = a.scale_log2;

  for (int it = 0; it < cnt; ++it) {
    const int64_t j = dense ? it : idx[it];
    const u32x4* kg = reinterpret_cast<const u32x4*>(kb + j * kTileBytes);
    const u32x4* vg = reinterpret_cast<const u32x4*>(vb + j * kTileBytes);
    u32x4 kr[8], vr[8];
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
      kr[mm] = kg[tid + 256 * mm];
      vr[mm] = vg[tid + 256 * mm];
    }
    __syncthreads();   // the previous block's K/V are no longer read
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
      const int L = tid + 256 * mm;
      *reinterpret_cast<u32x4*>(sK + swz(L >> 4, L & 15)) = kr[mm];
      *reinterpret_cast<u32x4*>(sV + swz(L >> 4, L & 15)) = vr[mm];
    }
    __syncthreads();

    // S^T: lane holds query l32, keys 32*kt + 8*(r/4) + 4*hl + r%4.
    f32x16 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.0f;
      const int key = 32 * kt + l32;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(sK + swz(key, 2 * st + hl));
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[st], s[kt], 0, 0, 0);
      }
    }

    // Online softmax (log2 domain).
    float mx = s[0][0];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    float rs = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r], c, -m_new));
        s[kt][r] = p;
        rs += p;
      }
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

    // P^T as B operand: slot (hl, e) of k-step (kt, ks) is key
    // 32*kt + 16*ks + 8*(e/4) + 4*hl + e%4, i.e. registers 8*ks .. 8*ks+7.
    bf16x8 pf[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[kt][ks][e] = (__bf16)s[kt][8 * ks + e];

    // O^T += V^T P^T; A operand: row d, the same permuted keys.
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 32 * db + l32;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int c0 = 4 * kt + 2 * ks;
          const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(sV + swz(d, c0) + 8 * hl);
          const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(sV + swz(d, c0 + 1) + 8 * hl);
          const bf16x8 va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[kt][ks], o[db], 0, 0, 0);
        }
    }
  }

  // Epilogue: lane holds query qrow, channels 32*db + 8*g4 + 4*hl + (0..3).
  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  uint16_t* ob = static_cast<uint16_t*>(a.o_t) + row * kTileElems + qrow * kHeadDim;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[db][4 * g4 + e] * inv);
      *reinterpret_cast<bf16x4*>(ob + 32 * db + 8 * g4 + 4 * hl) = w;
    }
  if (a.lse != nullptr && hl == 0) {
    const float v = lt > 0.0f ? (m + __log2f(lt)) * 0.69314718055994530942f : -INFINITY;
    a.lse[row * kTileTokens + qrow] = v;
  }
}

}  // namespace

hipError_t launch_attention(const Geo& g, const AttnArgs& a, hipStream_t s) {
  const int64_t rows = g.bh * g.n_tiles;
  hipLaunchKernelGGL(k_attn_fwd, dim3((unsigned)rows), dim3(256), 0, s, g, a);
  return hipGetLastError();
}

}  // namespace ssta

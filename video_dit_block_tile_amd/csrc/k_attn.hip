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
// O^T += V^T P^T.  Each lane feeds key row kperm(lane) (bits 2 and 3 of the
// lane index swapped) into the S^T product, which makes every 8 output
// registers of a lane 8 consecutive keys; V arrives dim-major, so the matching
// A operand of the P.V product is one 16-byte LDS read of a V^T row.
// K and V^T tiles (32 KB each) are staged in LDS with a 16-byte-chunk XOR
// swizzle (chunk ^ row%16) so the MFMA operand reads are conflict-free.
// Schedule: the hardware deals workgroup ids round-robin over the 8 XCDs.
// The grid is laid out so that XCD x receives, head after head, the
// contiguous slice [x*c, (x+1)*c) of that head's query blocks (c = ceil(n/8)).
// All XCDs therefore work on the same one or two heads at any time, whose K
// and V (118 MB per head at the 720p 10 s shape) stay resident in the 256 MB
// MALL, while within an XCD neighbouring query blocks share most of their
// window blocks in that XCD's L2.
// Memory: the next kept block's K and V^T are fetched into registers while
// the current block is computed, so one global-memory round trip overlaps each
// block.  Each block is processed as two halves of 64 keys, which halves the
// live score registers and keeps two waves per SIMD without spills.
// Softmax: the running max is only raised when some query's max grows by more
// than 8 in the log2 domain (probabilities stay below 2^8), so the O rescale
// is skipped on most blocks; the denominator is summed from the bf16-rounded
// probabilities with v_dot2 (the same weights the P.V product uses).
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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kTileBytes = kTileTokens * kHeadDim * 2;   // 32 KB
constexpr int kHalfBytes = kTileBytes / 2;               // 16 KB: 64 keys of K or V^T
constexpr unsigned kWaitVm0 = 0x0F70;                    // s_waitcnt vmcnt(0)
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// K half slot: 64 key rows of 256 B; 16-byte chunk c of row r sits at chunk c ^ (r % 16).
__device__ __forceinline__ int swz_k(int row, int chunk) {
  return row * 256 + ((chunk ^ (row & 15)) << 4);
}
// V^T half slot: 128 channel rows of 128 B (64 keys); chunk c of row d sits at
// chunk c ^ ((d / 2) % 8), so 16 consecutive rows read the same chunk from 16
// distinct bank groups.
__device__ __forceinline__ int swz_v(int d, int chunk) {
  return d * 128 + ((chunk ^ ((d >> 1) & 7)) << 4);
}

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return fmaxf(a, fmaxf(b, c));
}

// Lanes l and l^32 hold the two halves of one query's keys.  v_permlane32_swap
// with the value as both operands leaves {own, partner} in the two results (in
// an order that depends on the half), so their max and sum are the pair's.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Direct global->LDS loads (global_load_lds_dwordx4) of half h of one block.
// Each of the 4 waves issues 4 instructions of 1 KB; lane i of an instruction
// lands at byte 16*i of its 1 KB destination block, so the source address of
// each lane is chosen to put the right chunk there.  The per-lane byte offsets
// depend only on the lane and wave (computed once); the block base is uniform,
// so the loads use a scalar base plus a 32-bit lane offset.
struct DmaOffsets {
  uint32_t k[4], v[4];
};

__device__ __forceinline__ DmaOffsets dma_offsets(int wave, int lane) {
  DmaOffsets o;
#pragma unroll
  for (int mm = 0; mm < 4; ++mm) {
    const int b = 4 * wave + mm;
    const int row = 4 * b + (lane >> 4);            // K: rows 4b .. 4b+3 of the half
    o.k[mm] = row * 256 + (((lane & 15) ^ (row & 15)) << 4);
    const int d = 8 * b + (lane >> 3);              // V^T: channel rows 8b .. 8b+7
    o.v[mm] = d * 256 + (((lane & 7) ^ ((d >> 1) & 7)) << 4);
  }
  return o;
}

// K half h of the block at `tile`: rows 64h .. 64h+63 (16 KB contiguous).
__device__ __forceinline__ void dma_k_half(lds_u8* dst, const uint8_t* tile, int h, int wave,
                                           const DmaOffsets& off) {
  const uint8_t* base = tile + h * kHalfBytes;
#pragma unroll
  for (int mm = 0; mm < 4; ++mm)
    __builtin_amdgcn_global_load_lds(base + off.k[mm], dst + (4 * wave + mm) * 1024, 16, 0, 0);
}
// V^T half h of the block at `tile`: bytes 128h .. 128h+127 of each of the 128 rows.
__device__ __forceinline__ void dma_v_half(lds_u8* dst, const uint8_t* tile, int h, int wave,
                                           const DmaOffsets& off) {
  const uint8_t* base = tile + h * 128;
#pragma unroll
  for (int mm = 0; mm < 4; ++mm)
    __builtin_amdgcn_global_load_lds(base + off.v[mm], dst + (4 * wave + mm) * 1024, 16, 0, 0);
}

// Token index of the first token of block j within one (batch, head).
__device__ __forceinline__ int64_t block_origin(const Geo& g, int64_t j) {
  const int64_t bt = j / ((int64_t)g.ny * g.nx), by = (j / g.nx) % g.ny, bx = j % g.nx;
  return ((bt * g.tt) * g.H + by * g.th) * (int64_t)g.W + bx * g.tw;
}

// Token offset (from the block's first token) of in-block position r; block
// sizes are powers of two because their product is 128.
__device__ __forceinline__ uint32_t in_block_offset(const Geo& g, int r) {
  const int ltw = __builtin_ctz(g.tw), lth = __builtin_ctz(g.th);
  const int it = r >> (ltw + lth), iy = (r >> ltw) & (g.th - 1), ix = r & (g.tw - 1);
  return (uint32_t)((it * g.H + iy) * g.W + ix);
}



// kTok: Q and O are token-major [B, h, T*H*W, 128] (the query block is
// gathered and the output scattered directly); otherwise they are tile-major
// [B, h, n_tiles, 128, 128].  K is always tile-major: each K block is re-read
// by every query block that keeps it, so it pays to store it contiguously.
template <bool kTok>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void k_attn_fwd(Geo g, AttnArgs a, int64_t slice) {
  // Two-slot rings of half blocks: K slots at 0 and 16 KB, V^T slots at 32 and 48 KB.
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * kHalfBytes];

  // Head-synchronous XCD slices (see the file comment).
  const int64_t bid = blockIdx.x;
  const int64_t xcd = bid & 7, k8 = bid >> 3;
  const int64_t bh = k8 / slice;
  const int64_t qi = xcd * slice + (k8 - bh * slice);
  if (qi >= g.n_tiles) return;
  const int64_t row = bh * g.n_tiles + qi;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int kperm = (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  constexpr int64_t kTileElems = kTileTokens * kHeadDim;

  // qb: this lane's query row is qb + (kTok ? 0 : qrow * 128).
  const uint16_t* qb = static_cast<const uint16_t*>(a.q_t) + row * kTileElems;
  if (kTok) {
    // bh * N tokens precede this head; each lane reads its own query row.
    const uint16_t* qhead = static_cast<const uint16_t*>(a.q_t) + bh * g.N * kHeadDim;
    qb = qhead + (block_origin(g, qi) + in_block_offset(g, wave * 32 + (lane & 31))) * kHeadDim;
  }
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
    qf[s] = *reinterpret_cast<const bf16x8*>(qb + (kTok ? 0 : qrow * kHeadDim) + 16 * s + 8 * hl);

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m = -INFINITY;   // running (possibly stale) max of the log2-scaled scores
  float l = 0.0f;        // this lane's part of the running denominator
  const float c = a.scale_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Units u = 2*(list position) + half; unit u uses slot u % 2.
  const int units = 2 * cnt;
  const DmaOffsets doff = dma_offsets(wv, lane);
  if (units > 0) {
    const int64_t j0 = dense ? 0 : idx[0];
    dma_k_half((lds_u8*)smem, kb + j0 * kTileBytes, 0, wv, doff);
    dma_v_half((lds_u8*)(smem + 2 * kHalfBytes), vb + j0 * kTileBytes, 0, wv, doff);
  }

  for (int u = 0; u < units; ++u) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);   // this wave's loads of unit u have landed
    __syncthreads();                        // ... every wave's; and unit u-1 is done
    const int slot = u & 1;
    if (u + 1 < units) {                    // unit u+1 travels while unit u is computed
      const int un = u + 1;
      const int64_t jn = dense ? (un >> 1) : idx[un >> 1];
      dma_k_half((lds_u8*)(smem + (1 - slot) * kHalfBytes), kb + jn * kTileBytes, un & 1, wv,
                 doff);
      dma_v_half((lds_u8*)(smem + (3 - slot) * kHalfBytes), vb + jn * kTileBytes, un & 1, wv,
                 doff);
    }
    const uint8_t* sK = smem + slot * kHalfBytes;
    const uint8_t* sV = smem + (2 + slot) * kHalfBytes;

    // S^T for the unit's 64 keys: the A operand row of lane l32 is key kperm(l32)
    // (bits 2 and 3 of l32 swapped), so output register r of lane (l32, hl) holds
    // query l32 and key 32*t + 16*(r/8) + 8*hl + r%8 of the unit: each group of 8
    // registers is 8 consecutive keys.
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = 0.0f;
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(sK + swz_k(32 * t + kperm, 2 * st + hl));
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[st], s[t], 0, 0, 0);
      }

    // Online softmax in the log2 domain: the max is raised only when it grows by > 8.
    float mq[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float x = max3f(s[t][0], s[t][1], s[t][2]);
      x = max3f(x, s[t][3], s[t][4]);
      x = max3f(x, s[t][5], s[t][6]);
      x = max3f(x, s[t][7], s[t][8]);
      x = max3f(x, s[t][9], s[t][10]);
      x = max3f(x, s[t][11], s[t][12]);
      x = max3f(x, s[t][13], s[t][14]);
      mq[t] = fmaxf(x, s[t][15]);
    }
    float mx = fmaxf(mq[0], mq[1]);
    mx = pair_max(mx) * c;
    if (__any(mx > m + 8.0f)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m = m_new;
    }

    // P^T as B operand of k-step (t, ks): registers 8*ks .. 8*ks+7, which are
    // keys 32*t + 16*ks + 8*hl + (0..7) of the unit.  The denominator sums the
    // bf16-rounded probabilities (the weights the P.V product uses) with v_dot2.
    bf16x8 pf[2][2];
    float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pf[t][ks][e] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[t][8 * ks + e], c, -m));
        const bf16x8 v = pf[t][ks];
        l0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), ones, l0, false);
        l1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), ones, l1, false);
        l0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), ones, l0, false);
        l1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), ones, l1, false);
      }
    l += l0 + l1;

    // O^T += V^T P^T; A operand: row d of V^T, the same 8 consecutive keys
    // (chunk 4*t + 2*ks + hl of the unit's 64 keys).
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(
              sV + swz_v(32 * db + l32, 4 * t + 2 * ks + hl));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[t][ks], o[db], 0, 0, 0);
        }
  }

  // Epilogue: lane holds query qrow, channels 32*db + 8*g4 + 4*hl + (0..3).
  const float lt = pair_sum(l);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  uint16_t* ob = static_cast<uint16_t*>(a.o_t) + row * kTileElems + qrow * kHeadDim;
  if (kTok)
    ob = static_cast<uint16_t*>(a.o_t) +
         (bh * g.N + block_origin(g, qi) + in_block_offset(g, qrow)) * kHeadDim;
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
  const int64_t slice = (g.n_tiles + 7) / 8;
  const int64_t blocks = g.bh * slice * 8;
  if (a.token_io)
    hipLaunchKernelGGL(k_attn_fwd<true>, dim3((unsigned)blocks), dim3(256), 0, s, g, a, slice);
  else
    hipLaunchKernelGGL(k_attn_fwd<false>, dim3((unsigned)blocks), dim3(256), 0, s, g, a, slice);
  return hipGetLastError();
}

}  // namespace ssta

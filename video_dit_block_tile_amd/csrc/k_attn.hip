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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kTileBytes = kTileTokens * kHeadDim * 2;   // 32 KB

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 256 + ((chunk ^ (row & 15)) << 4);
}

// Loads one 32 KB tile (K or V^T) of block j into registers: 8 x 16 B per thread.
__device__ __forceinline__ void fetch_tile(u32x4 (&r)[8], const uint8_t* base, int64_t j,
                                           int tid) {
  const uint8_t* tile = base + j * kTileBytes;     // uniform across the workgroup
  const uint32_t off = (uint32_t)tid * 16u;
#pragma unroll
  for (int mm = 0; mm < 8; ++mm)
    r[mm] = *reinterpret_cast<const u32x4*>(tile + off + 4096u * mm);
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

__device__ __forceinline__ void stage_tile(uint8_t* lds, const u32x4 (&r)[8], int tid) {
#pragma unroll
  for (int mm = 0; mm < 8; ++mm) {
    const int L = tid + 256 * mm;
    *reinterpret_cast<u32x4*>(lds + swz(L >> 4, L & 15)) = r[mm];
  }
}

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return fmaxf(a, fmaxf(b, c));
}

// kTok: Q and O are token-major [B, h, T*H*W, 128] (the query block is
// gathered and the output scattered directly); otherwise they are tile-major
// [B, h, n_tiles, 128, 128].  K is always tile-major: each K block is re-read
// by every query block that keeps it, so it pays to store it contiguously.
template <bool kTok>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void k_attn_fwd(Geo g, AttnArgs a, int64_t slice) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kTileBytes];
  uint8_t* sK = smem;                 // [key][256 B]
  uint8_t* sV = smem + kTileBytes;    // [d][256 B]

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
  constexpr int64_t kTileElems = kTileTokens * kHeadDim;

  // qb: this lane's query row is qb + (kTok ? 0 : qrow * 128).
  const uint16_t* qb = static_cast<const uint16_t*>(a.q_t) + row * kTileElems;
  const uint8_t* kb = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(a.k_t) +
                                                       bh * g.n_tiles * kTileElems);
  if (kTok) {
    // bh * N tokens precede this head; each lane reads its own query row.
    const uint16_t* qhead = static_cast<const uint16_t*>(a.q_t) + bh * g.N * kHeadDim;
    qb = qhead + (block_origin(g, qi) + in_block_offset(g, wave * 32 + (lane & 31))) * kHeadDim;
  }
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

  u32x4 kr[8], vr[8];
  if (cnt > 0) {
    const int64_t j0 = dense ? 0 : idx[0];
    fetch_tile(kr, kb, j0, tid);
    fetch_tile(vr, vb, j0, tid);
  }

  for (int it = 0; it < cnt; ++it) {
    __syncthreads();   // every wave is done reading the previous block's K and V^T
    stage_tile(sK, kr, tid);
    stage_tile(sV, vr, tid);
    __syncthreads();
    if (it + 1 < cnt) {   // next block's K and V^T travel while this one is computed
      const int64_t jn = dense ? it + 1 : idx[it + 1];
      fetch_tile(kr, kb, jn, tid);
      fetch_tile(vr, vb, jn, tid);
    }

    // Two halves of 64 keys each; the lazily raised max makes them independent.
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      // S^T: the A operand row of lane l32 is key kperm(l32) (bits 2 and 3 of l32
      // swapped), so output register r of lane (l32, hl) holds query l32 and key
      // 32*kt + 16*(r/8) + 8*hl + r%8, kt = 2*hb + t: each group of 8 registers is
      // 8 consecutive keys.
      f32x16 s[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[t][r] = 0.0f;
#pragma unroll
      for (int st = 0; st < 8; ++st)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int key = 32 * (2 * hb + t) + kperm;
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(sK + swz(key, 2 * st + hl));
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
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * c;
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

      // P^T as B operand of k-step (kt, ks): registers 8*ks .. 8*ks+7, which are
      // keys 32*kt + 16*ks + 8*hl + (0..7).  The denominator sums the
      // bf16-rounded probabilities (the weights the P.V product uses) with v_dot2.
      bf16x8 pf[2][2];
      float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pf[t][ks][e] =
                (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[t][8 * ks + e], c, -m));
          const bf16x8 v = pf[t][ks];
          l0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), ones, l0, false);
          l1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), ones, l1, false);
          l0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), ones, l0, false);
          l1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), ones, l1, false);
        }
      l += l0 + l1;

      // O^T += V^T P^T; A operand: row d, the same permuted keys.
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            // A operand: row d of V^T, the same 8 consecutive keys (one 16-byte chunk).
            const int d = 32 * db + l32;
            const bf16x8 va = *reinterpret_cast<const bf16x8*>(
                sV + swz(d, 4 * (2 * hb + t) + 2 * ks + hl));
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[t][ks], o[db], 0, 0, 0);
          }
    }
  }

  // Epilogue: lane holds query qrow, channels 32*db + 8*g4 + 4*hl + (0..3).
  const float lt = l + __shfl_xor(l, 32);
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

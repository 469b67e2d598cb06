// Gradients of Step 4's block-sparse attention with the kept lists held fixed
// ("HunyuanVideo 1.5 Technical Report" summary page, section "SSTA: Selective
// and Sliding Tile Attention": the attention equation, Step 4, and the
// paragraph on integrating SSTA while the model is trained during
// distillation).  For a query token a and a kept key token b,
//   p_ab = exp(s_ab - lse_a),  D_a = dO_a . O_a,
//   dS_ab = p_ab (dO_a . v_b - D_a),
//   dq_a = scale sum_b dS_ab k_b,  dk_b = scale sum_a dS_ab q_a,
//   dv_b = sum_a p_ab dO_a,
// with lse_a the forward's log-sum-exp, so the probabilities are recomputed
// exactly instead of with a running max.
//
// gfx950 design.  Two kernels, each one workgroup of kR/32 waves per block
// and the matrix-core layouts of the forward kernel (v_mfma_f32_32x32x16_bf16;
// a lane feeds row kperm(lane) of the A operand, bits 2 and 3 swapped, so
// every 8 output registers are 8 consecutive rows and feed the next product
// as its B operand straight from registers):
//   k_attn_bwd_dq    per query block, over its kept key blocks in units of 32
//                    keys: S^T = K Q^T and dP^T = V dO^T (Q, dO of the wave's
//                    32 queries held in registers), dS^T in registers, then
//                    dQ^T += K^T dS^T with K^T read transposed from the K rows;
//   k_attn_bwd_dkdv  per key block, over the query blocks that keep it, in
//                    units of 32 queries, two waves per group of 32 keys: a V
//                    wave forms S = Q K^T (the keys held in registers), P and
//                    dV^T += dO^T P, and hands P to a K wave, which forms
//                    dP = dO V^T (the values held in registers),
//                    dS = P (dP - D) and dK^T += Q^T dS one unit later.
// The transposed operands (K^T, dO^T, Q^T: channel d of 8 consecutive rows)
// come from the same token rows in LDS through the transposing reads
// (ds_read_b64_tr_b16), so nothing is copied to a dim-major layout first.
// Both kernels run two waves per SIMD.  Every streamed unit (token rows
// gathered from token-major memory and the per-query lse*log2 e and D values)
// goes straight into LDS with buffer_load_dwordx4 ... lds into a ring of
// slots (two in k_attn_bwd_dq, three in k_attn_bwd_dkdv), as in the forward
// kernel.
//
// Algorithmic work per kept (query block, key block) pair: five 128^3
// products (S, dP, dQ, dK, dV) = 21.0 MFLOP; the two kernels compute S and dP
// once each more, 29.4 MFLOP executed.
//
// Joint video + text sequences: blocks from n_tiles on are text blocks of
// consecutive tokens after the clip's.  A clip query block keeps its list and
// every text block, a text query block keeps every block; so a clip key
// block is kept by the query blocks of its transposed list and every text
// query block, and a text key block by every query block.
#include "ssta_internal.h"

namespace ssta {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kUnitBytes = 8192;                          // 32 token rows
// Blocks hold kR = 128 or 64 tokens: a workgroup has kR/32 waves (32 rows of
// the block each) and streams the other side in kR/32 units of 32 per block.
template <int kR>
struct Blk {
  static constexpr int kWaves = kR / 32;
  static constexpr int kLoads = 8 / kWaves;           // 1 KB loads per wave per 8 KB unit
  static constexpr int kUnits = kR / 32;              // 32-row units per block
  static constexpr int kBytes = kR * kHeadDim * 2;    // one block of one tensor
};
constexpr unsigned kWaitVm0 = 0x0F70;                     // s_waitcnt vmcnt(0)
constexpr float kLog2e = 1.44269504088896340736f;

// Unit of 32 token rows (256 B each): 16-byte chunk c of row r sits at chunk
// c ^ row_swz(r), row_swz(r) = 4*(r % 4) + (r / 4) % 4 (the two 2-bit fields of
// r's low nibble swapped).  A unit is read two ways, both conflict-free: a
// whole chunk per lane from 16 consecutive rows (a bijection on the low
// nibble), and 8 bytes per lane from 4 consecutive rows by the transposing
// reads (row_swz's upper bits differ across any 4 aligned rows).
__device__ __forceinline__ int row_swz(int row) {
  return ((row & 3) << 2) | ((row >> 2) & 3);
}
__device__ __forceinline__ int swz_row(int row, int chunk) {
  return row * 256 + ((chunk ^ row_swz(row)) << 4);
}

// The transposed operand from a row unit: for k-step ks and channel block db
// lane (l32, hl) needs channel 32*db + l32 of the 8 rows 16ks + 8hl + (0..7),
// which two transposing reads (ds_read_b64_tr_b16) give: within each group of
// 16 lanes, lane j reads 4 channels (8 B) of row j/4 of a 4-row group, and
// lane i receives channel i of those 4 rows.  row_t_base is this lane's byte
// offset for ks = 0, db = 0 and the first 4 rows; channel block db flips bits
// 6-7 (db << 6), the second 4 rows lie at (offset + 1 KB) ^ 16, and k-step ks
// adds 16 rows (4 KB).
__device__ __forceinline__ int row_t_base(int lane) {
  const int j = lane & 15, grp = (lane >> 4) & 1, hl = lane >> 5;
  const int kq = j >> 2;                         // row within the 4-row group
  const int row = 8 * hl + kq;
  const int chunk = (2 * grp + ((j & 3) >> 1)) ^ row_swz(row);   // channel chunk 2grp + ..
  return row * 256 + chunk * 16 + 8 * (j & 1);
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ bf16x8 row_t_operand(const uint8_t* unit, int tb, int ks, int db) {
  const int o0 = (tb ^ (db << 6)) + 4096 * ks;
  const int o1 = ((tb + 1024) ^ 16 ^ (db << 6)) + 4096 * ks;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(unit + o0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(unit + o1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// (lse * log2 e, D) of query r of block row `row` (R queries per block):
// each group of 32 queries holds their 32 lse values, then their 32 D values,
// so a dK/dV wave reads only the half it uses.
__device__ __forceinline__ int64_t ld_index(int64_t row, int r, int R) {
  return row * 2 * R + (r >> 5) * 64 + (r & 31);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Per-lane source offsets of this wave's 1 KB loads of a row unit, for a
// workgroup of kW waves that shares the unit's eight 1 KB loads.
template <int kR, int kW = Blk<kR>::kWaves>
struct UnitOffsets {
  static constexpr int kLoads = 8 / kW;
  uint32_t rows[kLoads];
};
template <int kR, int kW = Blk<kR>::kWaves>
__device__ __forceinline__ UnitOffsets<kR, kW> unit_offsets(const Geo& g, int wave, int lane) {
  UnitOffsets<kR, kW> o;
#pragma unroll
  for (int mm = 0; mm < o.kLoads; ++mm) {
    const int b = o.kLoads * wave + mm;            // 1 KB destination block 0..7
    const int row = 4 * b + (lane >> 4);           // token rows 4b .. 4b+3
    o.rows[mm] = in_block_offset(g, row) * 256 + (((lane & 15) ^ row_swz(row)) << 4);
  }
  return o;
}
// Which of positions 32p .. 32p+31 of block j exist: all of them unless the
// block is an edge block of a ragged grid or the last, partial text block.
// kGen: the kernels' instance for ragged grids and joint text; the other one
// (grids the block size divides, no text) compiles every such check away.
template <bool kGen, int kR>
__device__ __forceinline__ uint32_t rows_valid(const Geo& g, uint32_t j, int p, int lane) {
  if (!kGen) return ~0u;
  if (j >= g.n_tiles) {
    const int64_t u0 = (j - g.n_tiles) * kR + 32 * p;   // first text token
    if (u0 + 32 <= g.L) return ~0u;
    return (uint32_t)__ballot(u0 + (lane & 31) < g.L);
  }
  if (!g.ragged) return ~0u;
  const BlockExtent e = block_extent(g, j);
  if (e.full) return ~0u;
  return (uint32_t)__ballot(pos_exists(g, e, 32 * p + (lane & 31)));
}

// Rows 32p .. 32p+31 of block j, gathered from token-major memory.  A row
// whose position does not exist (bit clear in `valid`) is read from the
// block's first token instead, so every score it enters stays bounded by
// the row's log-sum-exp; the kernels zero its dS or P, so it adds nothing.
// A text block's rows are consecutive tokens.
template <bool kGen, int kR, int kW = Blk<kR>::kWaves>
__device__ __forceinline__ void dma_rows(uint8_t* dst, __amdgpu_buffer_rsrc_t rs, const Geo& g,
                                         uint32_t j, uint32_t clip_origin, int p, int wave,
                                         int lane, uint32_t valid,
                                         const UnitOffsets<kR, kW>& off) {
  constexpr int kL = UnitOffsets<kR, kW>::kLoads;
  if (!kGen || (j < g.n_tiles && valid == ~0u)) {
    // a clip block's unit with every row: one straight path, the same in both
    // instances (the general one below handles text blocks and missing rows)
    const uint32_t so = clip_origin * 256u + in_block_offset(g, 32 * p) * 256u;
#pragma unroll
    for (int mm = 0; mm < kL; ++mm)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_u8*)(dst + (kL * wave + mm) * 1024), 16,
                                               off.rows[mm], so, 0, 0);
    return;
  }
  const bool part = valid != ~0u;
  const bool text = j >= g.n_tiles;
  const uint32_t origin = text ? (uint32_t)(g.N + (j - g.n_tiles) * kR) : clip_origin;
  const uint32_t half = (text ? 32u * p : in_block_offset(g, 32 * p)) * 256u;
  const uint32_t so = origin * 256u + (part ? 0u : half);
#pragma unroll
  for (int mm = 0; mm < kL; ++mm) {
    const int r = 4 * (kL * wave + mm) + (lane >> 4);
    uint32_t vo = text ? r * 256 + (((lane & 15) ^ row_swz(r)) << 4) : off.rows[mm];
    if (part) vo = ((valid >> r) & 1u) ? vo + half : (vo & 255u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_u8*)(dst + (kL * wave + mm) * 1024), 16,
                                             vo, so, 0, 0);
  }
}

// Token (within its head) of position r of block j, or of the block's first
// position when r does not exist.
template <bool kGen, int kR>
__device__ __forceinline__ int64_t row_token(const Geo& g, int64_t j, int r, bool exists) {
  if (kGen && j >= g.n_tiles) return g.N + (j - g.n_tiles) * kR + (exists ? r : 0);
  return block_first_token(g, (uint32_t)j) + (exists ? in_block_offset(g, r) : 0u);
}

// The blocks a row runs over, 64 at a time: lane i holds list position
// base + i, which is the caller's id (clamped to the clip's blocks) below
// `listed` and, in the kGen instance, text block n_tiles + (pos - listed)
// after it; in a dense list position i is block i.  With each id the first
// token of the block (clip blocks) and, in the kGen instance, a ballot of
// which of the 64 are clip blocks holding every position, so that a unit's
// set-up is two v_readlane and a bit test; positions are requested in
// non-decreasing order.
template <bool kGen>
struct IdStream {
  const int32_t* idx;
  int listed, base, ids;
  uint32_t org;
  uint64_t whole;
  bool dense;
  __device__ __forceinline__ void fill(const Geo& g, int lane) {
    const int pos = base + lane;
    const int last = (int)g.n_tiles - 1;
    // a caller's id outside the clip's blocks is clamped to one, so a
    // malformed list reads only the head's own blocks
    ids = dense ? pos
                : (pos < listed ? min(max(idx[pos], 0), last)
                                : (kGen ? (int)g.n_tiles + (pos - listed) : 0));
    org = block_origin32(g, (uint32_t)min(ids, last));
    if (kGen)
      whole = __ballot(ids <= last &&
                       (!g.ragged || block_extent(g, (uint32_t)min(ids, last)).full));
  }
  __device__ __forceinline__ void init(const Geo& g, const int32_t* p, int n, bool d, int lane) {
    idx = p; listed = n; dense = d; base = 0;
    fill(g, lane);
  }
  // block at list position pos; origin: its first token (clip blocks);
  // full: a clip block with every position (always, outside kGen)
  __device__ __forceinline__ uint32_t at(const Geo& g, int pos, int lane, uint32_t& origin,
                                         bool& full) {
    if (pos >= base + 64) {
      base += 64;
      fill(g, lane);
    }
    origin = (uint32_t)__builtin_amdgcn_readlane((int)org, pos - base);
    full = !kGen || ((whole >> (pos - base)) & 1u);
    return dense ? (uint32_t)pos : (uint32_t)__builtin_amdgcn_readlane(ids, pos - base);
  }
};

// Token-major row of token `tok` as 8 B operands of a 32x32x16 product:
// channels 16*s + 8*hl .. +8.
__device__ __forceinline__ void load_row_operand(bf16x8 (&f)[8], const uint16_t* row, int hl) {
#pragma unroll
  for (int s = 0; s < 8; ++s) f[s] = *reinterpret_cast<const bf16x8*>(row + 16 * s + 8 * hl);
}

// Writes a [128 ch x 32 tok] fp32 accumulator (lane: token l32, channels
// 32*db + 8*g4 + 4*hl + 0..3) times `mul` as bf16 into the token's row.
__device__ __forceinline__ void store_row(uint16_t* row, const f32x16 (&acc)[4], float mul,
                                          int hl) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[db][4 * g4 + e] * mul);
      *reinterpret_cast<bf16x4*>(row + 32 * db + 8 * g4 + 4 * hl) = w;
    }
}

// ------------------------------------------------------------------ dQ

template <bool kGen, int kR>
__global__ __launch_bounds__(kR * 2) __attribute__((amdgpu_waves_per_eu(2)))
void k_attn_bwd_dq(Geo g, BwdArgs a, AttnGrid grid) {
  constexpr int kUnits = Blk<kR>::kUnits;
  // slot s (16 KB): K rows | V rows of one 32-key unit
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * kUnitBytes];
  int64_t bh, qi;
  if (!attn_block<kGen>(g, grid, blockIdx.x, bh, qi)) return;
  const int64_t row = bh * g.n_rows + qi;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int kperm = (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  const int qrow = 32 * wv + l32;
  const int64_t head = bh * g.S;
  // a query position its block lacks reads the block's first token and
  // stores nothing
  const bool qvalid = (rows_valid<kGen, kR>(g, (uint32_t)qi, wv, lane) >> l32) & 1u;
  const int64_t qtok = head + row_token<kGen, kR>(g, qi, qrow, qvalid);

  bf16x8 qf[8], df[8];
  load_row_operand(qf, static_cast<const uint16_t*>(a.q) + qtok * kHeadDim, hl);
  load_row_operand(df, static_cast<const uint16_t*>(a.dout) + qtok * kHeadDim, hl);
  const float lse2 = a.ld[ld_index(row, qrow, kR)];
  const float dq_d = a.ld[ld_index(row, qrow, kR) + 32];
  const float c = a.scale_log2;

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  // key blocks: the kept list, then every text block; a text query block
  // (or dense attention) takes every block
  const bool all_blocks = a.kv_cnt == nullptr || (kGen && qi >= g.n_tiles);
  const int64_t kvrow = bh * g.n_tiles + qi;
  const int listed = all_blocks ? 0 : min(max(a.kv_cnt[kvrow], 0), a.max_kept);
  const int cnt = all_blocks ? (int)g.n_rows : listed + (kGen ? g.n_txt : 0);
  IdStream<kGen> ids;
  ids.init(g, all_blocks ? nullptr : a.kv_idx + kvrow * a.max_kept, listed, all_blocks, lane);
  const UnitOffsets<kR> off = unit_offsets<kR>(g, wv, lane);
  const int tb = row_t_base(lane);
  // token-major: S rows of 256 B per head
  const int64_t tok_bytes = g.S * (int64_t)(kHeadDim * 2);
  const __amdgpu_buffer_rsrc_t krs = rsrc(static_cast<const uint16_t*>(a.k) + head * kHeadDim,
                                          tok_bytes);
  const __amdgpu_buffer_rsrc_t vrs = rsrc(static_cast<const uint16_t*>(a.v) + head * kHeadDim,
                                          tok_bytes);
  // returns which of the unit's 32 keys exist
  auto load_unit = [&](int u, uint8_t* dst) -> uint32_t {
    uint32_t org;
    bool full;
    const uint32_t j = ids.at(g, u / kUnits, lane, org, full);
    const int p = u % kUnits;
    const uint32_t valid = full ? ~0u : rows_valid<kGen, kR>(g, j, p, lane);
    dma_rows<kGen, kR>(dst, krs, g, j, org, p, wv, lane, valid, off);
    dma_rows<kGen, kR>(dst + kUnitBytes, vrs, g, j, org, p, wv, lane, valid, off);
    return valid;
  };

  const int units = kUnits * cnt;
  uint32_t valid_next = ~0u;
  if (units > 0) valid_next = load_unit(0, smem);
  for (int u = 0; u < units; ++u) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    uint8_t* cur = smem + (u & 1) * 2 * kUnitBytes;
    const uint32_t valid = valid_next;
    if (u + 1 < units) valid_next = load_unit(u + 1, smem + ((u + 1) & 1) * 2 * kUnitBytes);
    const uint8_t* sK = cur;
    const uint8_t* sV = cur + kUnitBytes;

    // S^T and dP^T for the unit's 32 keys: register r of lane (l32, hl) is
    // query l32 and key 16*(r/8) + 8*hl + r%8.
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.0f;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(sK + swz_row(kperm, 2 * st + hl));
      const bf16x8 va = *reinterpret_cast<const bf16x8*>(sV + swz_row(kperm, 2 * st + hl));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[st], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df[st], dp, 0, 0, 0);
    }
    // dS^T = P^T (dP^T - D), as the B operand of k-step ks (keys 16*ks + 8*hl + e);
    // zero for a key its block lacks (its row holds the block's first token).
    bf16x8 dsf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * ks + e;
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lse2));
        dsf[ks][e] = (__bf16)(pr * (dp[r] - dq_d));
      }
    if (kGen && valid != ~0u)   // uniform: only units with missing keys
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (!((valid >> (16 * ks + 8 * hl + e)) & 1u)) dsf[ks][e] = (__bf16)0.0f;
    // dQ^T += K^T dS^T: A operand row d of K^T, the same 8 keys, read
    // transposed from the K rows.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 kt = row_t_operand(sK, tb, ks, db);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, dsf[ks], acc[db], 0, 0, 0);
      }
  }
  if (qvalid) store_row(static_cast<uint16_t*>(a.dq) + qtok * kHeadDim, acc, a.scale, hl);
}

// ------------------------------------------------------------------ dK, dV

// dV^T += dO^T P and dK^T += Q^T dS with dS = P (dP - D), one workgroup per key
// block, in units of 32 queries.  The block's keys form kR/32 groups of 32;
// each group has two waves:
//   a V wave: S = Q K^T (its keys' K rows held in registers), P, and
//             dV^T += dO^T P; it hands P (fp32) to its partner through LDS;
//   a K wave, one unit behind: dP = dO V^T (the keys' V rows in registers),
//             dS = P (dP - D) from the partner's P, and dK^T += Q^T dS.
// Each wave thus needs one accumulator and one operand block, so two waves
// share a SIMD, and each does 16 of the 32 products of a unit.  Iteration u:
// the V waves take unit u, the K waves unit u-1, and unit u+1 is loading:
// three slots of Q rows, dO rows and the units' lse*log2 e and D values, plus
// two P buffers.  The arithmetic (products, their order, the roundings) is
// the same as one wave doing both, so the gradients are too.
template <int kR>
struct DkdvShape {
  static constexpr int kGroups = kR / 32;             // 32-key groups per block
  static constexpr int kWaves = 2 * kGroups;
  static constexpr int kSlot = 2 * kUnitBytes + 256;  // Q rows | dO rows | 32 lse2 | 32 D
  static constexpr int kPBuf = kGroups * 64 * 64;     // 16 fp32 per lane per group
  static constexpr int kLds = 3 * kSlot + 2 * kPBuf;
};

template <bool kGen, int kR>
__global__ __launch_bounds__(DkdvShape<kR>::kWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void k_attn_bwd_dkdv(Geo g, BwdArgs a, AttnGrid grid) {
  using Sh = DkdvShape<kR>;
  constexpr int kUnits = Blk<kR>::kUnits;
  constexpr int kSlot = Sh::kSlot;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Sh::kLds];
  // text key blocks (kept by every query block) first; then, with the kept
  // lists, each head's key blocks longest first (k_order_blocks), dealt
  // round-robin over the XCDs; under dense attention, XCD slices
  int64_t bh, kj;
  if (a.order != nullptr && !(kGen && (int64_t)blockIdx.x < grid.text_wgs)) {
    const int64_t b = (int64_t)blockIdx.x - grid.text_wgs;
    bh = b / g.n_tiles;
    if (bh >= g.bh) return;
    kj = a.order[b];
  } else if (!attn_block<kGen>(g, grid, blockIdx.x, bh, kj)) {
    return;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool vwave = wv < Sh::kGroups;           // V wave (else K wave), uniform
  const int grp = vwave ? wv : wv - Sh::kGroups;
  const int l32 = lane & 31, hl = lane >> 5;
  const int kperm = (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  const int kr = 32 * grp + l32;                 // this lane's key within the block
  const int64_t head = bh * g.S;
  // a key position its block lacks reads the block's first token and stores
  // nothing
  const bool kvalid = (rows_valid<kGen, kR>(g, (uint32_t)kj, grp, lane) >> l32) & 1u;
  const int64_t ktok = head + row_token<kGen, kR>(g, kj, kr, kvalid);

  // B operand of the wave's score product: its 32 keys (V wave: S = Q K^T)
  // or their values (K wave: dP = dO V^T).
  bf16x8 bop[8];
  load_row_operand(bop, static_cast<const uint16_t*>(vwave ? a.k : a.v) + ktok * kHeadDim, hl);
  const float c = a.scale_log2;

  f32x16 acc[4];   // dV^T (V wave) or dK^T (K wave)
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  // query blocks that keep this key block: its transposed list, then every
  // text query block; every query block keeps a text key block (and all
  // keep all under dense attention)
  const bool all_blocks = a.q_cnt == nullptr || (kGen && kj >= g.n_tiles);
  const int64_t klist = bh * g.n_tiles + kj;
  const int listed = all_blocks ? 0 : a.q_cnt[klist];
  const int cnt = all_blocks ? (int)g.n_rows : listed + (kGen ? g.n_txt : 0);
  IdStream<kGen> ids;
  ids.init(g, all_blocks ? nullptr : a.q_idx + klist * a.q_width, listed, all_blocks, lane);
  const UnitOffsets<kR, Sh::kWaves> off = unit_offsets<kR, Sh::kWaves>(g, wv, lane);
  const int tb = row_t_base(lane);
  const int64_t tok_bytes = g.S * (int64_t)(kHeadDim * 2);
  const __amdgpu_buffer_rsrc_t qrs = rsrc(static_cast<const uint16_t*>(a.q) + head * kHeadDim,
                                          tok_bytes);
  const __amdgpu_buffer_rsrc_t drs = rsrc(static_cast<const uint16_t*>(a.dout) + head * kHeadDim,
                                          tok_bytes);
  const __amdgpu_buffer_rsrc_t lrs =
      rsrc(a.ld + bh * g.n_rows * kR * 2, g.n_rows * kR * 8);
  // returns which of the unit's 32 queries exist
  auto load_unit = [&](int u, uint8_t* dst) -> uint32_t {
    uint32_t org;
    bool full;
    const uint32_t i = ids.at(g, u / kUnits, lane, org, full);
    const int p = u % kUnits;
    const uint32_t valid = full ? ~0u : rows_valid<kGen, kR>(g, i, p, lane);
    dma_rows<kGen, kR, Sh::kWaves>(dst, qrs, g, i, org, p, wv, lane, valid, off);
    dma_rows<kGen, kR, Sh::kWaves>(dst + kUnitBytes, drs, g, i, org, p, wv, lane, valid, off);
    if (wv == 0 && lane < 16)   // the unit's 32 lse2 and 32 D values = 256 B
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          lrs, (lds_u8*)(dst + 2 * kUnitBytes), 16, (uint32_t)lane * 16,
          (i * (uint32_t)kR + 32u * p) * 8u, 0, 0);
    return valid;
  };
  auto slot = [&](int u) -> uint8_t* { return smem + (u % 3) * kSlot; };
  // P of unit u for this group: 16 fp32 per lane, lane-major float4s
  auto pbuf = [&](int u) -> f32x4* {
    return reinterpret_cast<f32x4*>(smem + 3 * kSlot + (u & 1) * Sh::kPBuf + grp * 4096) + lane;
  };
  constexpr int kAhead = 4;   // row operands requested ahead of their products

  const int units = kUnits * cnt;
  uint32_t v_next = ~0u, v_cur = ~0u, v_prev = ~0u;   // which queries of units u+1, u, u-1 exist
  if (units > 0) v_next = load_unit(0, slot(0));
  // Iteration u: the V waves take unit u from slot sv, the K waves unit u-1
  // from slot sk, and unit u+1 loads into slot sn (which held unit u-2).
  for (int u = 0; u <= units; ++u) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);   // this wave's loads of unit u have landed
    __syncthreads();                        // ... every wave's; units u-2 and P(u-2) are done
    v_prev = v_cur;
    v_cur = v_next;
    if (u + 1 < units) v_next = load_unit(u + 1, slot(u + 1));   // into unit u-2's slot
    const int w = vwave ? u : u - 1;         // the unit this wave takes
    if (w < 0 || w >= units) continue;
    const uint8_t* sQ = slot(w);
    const uint8_t* sD = sQ + kUnitBytes;
    // the wave's score product: S = Q K^T (V wave) or dP = dO V^T (K wave);
    // register r of lane (l32, hl) is key l32 and query 16*(r/8) + 8*hl + r%8
    const uint8_t* sA = vwave ? sQ : sD;
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.0f;
    bf16x8 ra[kAhead];
#pragma unroll
    for (int st = 0; st < kAhead; ++st)
      ra[st] = *reinterpret_cast<const bf16x8*>(sA + swz_row(kperm, 2 * st + hl));
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[st % kAhead], bop[st], sc, 0, 0, 0);
      const int n = st + kAhead;
      if (n < 8) ra[st % kAhead] = *reinterpret_cast<const bf16x8*>(sA + swz_row(kperm, 2 * n + hl));
    }
    // lse2 (V wave) or D (K wave) of the lane's 16 queries 16*ks + 8*hl + e:
    // lv[2*ks + e/4][e%4], from the unit's 32 lse2 values or the 32 D values
    // after them
    const f32x4* sL = reinterpret_cast<const f32x4*>(sQ + 2 * kUnitBytes) + (vwave ? 0 : 8);
    f32x4 lv[4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int x = 0; x < 2; ++x) lv[2 * ks + x] = sL[4 * ks + 2 * hl + x];
    const uint32_t valid = vwave ? v_cur : v_prev;
    bf16x8 bo[2];   // P (V wave) or dS (K wave) as the B operand of k-step ks
    if (vwave) {
      // P = exp2(S c - lse2); zero for a query its block lacks (its rows hold
      // the block's first token).  The fp32 values go to the K wave.
      f32x4 pv[4];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ks = r >> 3, e = r & 7;
        const float pr =
            __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], c, -lv[2 * ks + (e >> 2)][e & 3]));
        pv[r >> 2][r & 3] = pr;
        bo[ks][e] = (__bf16)pr;
      }
      if (kGen && valid != ~0u)   // uniform: only units with missing queries
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((valid >> (16 * (r >> 3) + 8 * hl + (r & 7))) & 1u)) {
            pv[r >> 2][r & 3] = 0.0f;
            bo[r >> 3][r & 7] = (__bf16)0.0f;
          }
      f32x4* pb = pbuf(w);
#pragma unroll
      for (int x = 0; x < 4; ++x) pb[64 * x] = pv[x];
    } else {
      // dS = P (dP - D) with the V wave's P of this unit
      const f32x4* pb = pbuf(w);
      f32x4 pv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) pv[x] = pb[64 * x];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ks = r >> 3, e = r & 7;
        bo[ks][e] = (__bf16)(pv[r >> 2][r & 3] * (sc[r] - lv[2 * ks + (e >> 2)][e & 3]));
      }
      if (kGen && valid != ~0u)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((valid >> (16 * (r >> 3) + 8 * hl + (r & 7))) & 1u)) bo[r >> 3][r & 7] = (__bf16)0.0f;
    }
    // dV^T += dO^T P (V wave) or dK^T += Q^T dS (K wave): A operand row d of
    // the same 8 queries, read transposed from the dO or Q rows.
    const uint8_t* sT = vwave ? sD : sQ;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_t_operand(sT, tb, ks, db), bo[ks],
                                                          acc[db], 0, 0, 0);
  }
  if (kvalid)
    store_row(static_cast<uint16_t*>(vwave ? a.dv : a.dk) + ktok * kHeadDim, acc,
              vwave ? 1.0f : a.scale, hl);
}

// ------------------------------------------------------------------ helpers

// (lse * log2 e, D = dO . O) per query, tile-major like the LSE: one
// workgroup per (batch*head, block) of 2*R threads, two threads per token (64
// channels each).
// A position an edge block of a ragged grid lacks gets the block's first
// query's lse and D = 0: the products then read that query in its place.
__global__ __launch_bounds__(256) void k_attn_bwd_prep(Geo g, const uint16_t* __restrict__ o,
                                                       const uint16_t* __restrict__ dout,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ ld) {
  const int64_t blk = blockIdx.x, bh = blk / g.n_rows, tile = blk % g.n_rows;
  const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
  const bool text = tile >= g.n_tiles;
  const BlockExtent ext = block_extent(g, text ? 0u : (uint32_t)tile);
  const bool exists =
      text ? (tile - g.n_tiles) * g.R + r < g.L : (ext.full || pos_exists(g, ext, r));
  if (!exists) {
    if (half == 0) {
      ld[ld_index(blk, r, g.R)] = lse[blk * g.R] * kLog2e;
      ld[ld_index(blk, r, g.R) + 32] = 0.0f;
    }
    return;
  }
  const int64_t tok =
      bh * g.S + (text ? g.N + (tile - g.n_tiles) * g.R + r
                       : block_first_token(g, (uint32_t)tile) + pos_token_offset(g, r));
  const uint16_t* orow = o + tok * kHeadDim + 64 * half;
  const uint16_t* drow = dout + tok * kHeadDim + 64 * half;
  float acc = 0.0f;
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const bf16x8 ov = *reinterpret_cast<const bf16x8*>(orow + 8 * x);
    const bf16x8 dv = *reinterpret_cast<const bf16x8*>(drow + 8 * x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)ov[e], (float)dv[e], acc);
  }
  acc += __shfl_xor(acc, 1);
  if (half == 0) {
    ld[ld_index(blk, r, g.R)] = lse[blk * g.R + r] * kLog2e;
    ld[ld_index(blk, r, g.R) + 32] = acc;
  }
}

// Zero fill of a word array (no memset, so the sequence can be captured).
__global__ __launch_bounds__(256) void k_fill_zero(uint32_t* __restrict__ p, int64_t words) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < words) p[i] = 0u;
}

// Transposed membership bits: mask_t[bh][j] has bit i set if query block i
// keeps key block j.
__global__ __launch_bounds__(256) void k_set_bits(Geo g, const int32_t* __restrict__ kv_idx,
                                                  const int32_t* __restrict__ kv_cnt,
                                                  int32_t max_kept, uint32_t* __restrict__ mask_t,
                                                  int64_t words) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t / max_kept, c = t % max_kept;
  if (row >= g.bh * g.n_tiles || c >= kv_cnt[row]) return;
  const int64_t bh = row / g.n_tiles, i = row % g.n_tiles;
  const int64_t j = kv_idx[row * max_kept + c];
  if (j < 0 || j >= g.n_tiles) return;   // not a clip block: no bit to set
  atomicOr(mask_t + (bh * g.n_tiles + j) * words + (i >> 5), 1u << (i & 31));
}

// Ascending query-block list of every key block from its bit row.
__global__ __launch_bounds__(256) void k_gather_lists(Geo g, const uint32_t* __restrict__ mask_t,
                                                      int64_t words, int32_t* __restrict__ q_idx,
                                                      int32_t* __restrict__ q_cnt) {
  const int64_t krow = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (krow >= g.bh * g.n_tiles) return;
  const uint32_t* bits = mask_t + krow * words;
  int32_t* out = q_idx + krow * g.n_tiles;
  int32_t m = 0;
  for (int64_t w = 0; w < words; ++w) {
    uint32_t x = bits[w];
    while (x) {
      const int b = __builtin_ctz(x);
      out[m++] = (int32_t)(w * 32 + b);
      x &= x - 1;
    }
  }
  q_cnt[krow] = m;
}

// Key blocks of every head in decreasing order of the number of query
// blocks that keep them (ties: ascending block id), for the dK/dV grids: a
// key block's workgroup runs over that many query blocks, and top-k
// selection makes a few key blocks many times more popular than the median.
// Taking the longest first, dealt round-robin over the XCDs, balances the
// XCDs and leaves only short workgroups for the end of the launch.  A
// counting sort per head (one workgroup): bucket b holds the count
// kOrderBuckets-1-b (counts beyond share the first bucket), and a block's
// place within its bucket is the number of earlier blocks with the same
// bucket, found chunk by chunk.
constexpr int kOrderBuckets = 4096;
constexpr int kOrderThreads = 1024;
__global__ __launch_bounds__(kOrderThreads) void k_order_blocks(Geo g,
                                                                const int32_t* __restrict__ q_cnt,
                                                                int32_t* __restrict__ order) {
  __shared__ uint32_t start[kOrderBuckets];
  __shared__ uint32_t part[kOrderThreads];
  __shared__ uint16_t chunk[kOrderThreads];
  const int t = threadIdx.x;
  const int64_t n = g.n_tiles;
  const int32_t* cnt = q_cnt + (int64_t)blockIdx.x * n;
  int32_t* out = order + (int64_t)blockIdx.x * n;
  auto bucket = [&](int64_t j) -> int {
    return kOrderBuckets - 1 - min(cnt[j], kOrderBuckets - 1);
  };
  for (int b = t; b < kOrderBuckets; b += kOrderThreads) start[b] = 0u;
  __syncthreads();
  for (int64_t j = t; j < n; j += kOrderThreads) atomicAdd(&start[bucket(j)], 1u);
  __syncthreads();
  // exclusive scan of the bucket sizes: 4 buckets per thread, then the
  // threads' totals
  constexpr int kPer = kOrderBuckets / kOrderThreads;
  uint32_t own = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) own += start[kPer * t + e];
  part[t] = own;
  __syncthreads();
  for (int d = 1; d < kOrderThreads; d *= 2) {
    const uint32_t add = t >= d ? part[t - d] : 0u;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  uint32_t run = part[t] - own;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const uint32_t c = start[kPer * t + e];
    start[kPer * t + e] = run;
    run += c;
  }
  __syncthreads();
  for (int64_t c0 = 0; c0 < n; c0 += kOrderThreads) {
    const int64_t j = c0 + t;
    const int b = j < n ? bucket(j) : -1;
    chunk[t] = (uint16_t)(b < 0 ? 0xFFFF : b);
    __syncthreads();
    if (b >= 0) {
      uint32_t before = 0;
      for (int i = 0; i < t; ++i) before += chunk[i] == (uint16_t)b;
      out[start[b] + before] = (int32_t)j;
    }
    __syncthreads();
    if (b >= 0) atomicAdd(&start[b], 1u);
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_attention_bwd_prep(const Geo& g, const void* o, const void* dout,
                                     const float* lse, float* ld, hipStream_t s) {
  hipLaunchKernelGGL(k_attn_bwd_prep, dim3((unsigned)(g.bh * g.n_rows)), dim3(2 * g.R), 0, s, g,
                     static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dout), lse,
                     ld);
  return hipGetLastError();
}

hipError_t launch_transpose_lists(const Geo& g, const int32_t* kv_idx, const int32_t* kv_cnt,
                                  int32_t max_kept, uint32_t* mask_t, int32_t* q_idx,
                                  int32_t* q_cnt, int32_t* order, hipStream_t s) {
  const int64_t rows = g.bh * g.n_tiles;
  const int64_t words = (g.n_tiles + 31) / 32;
  const int64_t total = rows * words;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, mask_t,
                     total);
  if (max_kept > 0) {
    const int64_t pairs = rows * max_kept;
    hipLaunchKernelGGL(k_set_bits, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0, s, g,
                       kv_idx, kv_cnt, max_kept, mask_t, words);
  }
  hipLaunchKernelGGL(k_gather_lists, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, g,
                     mask_t, words, q_idx, q_cnt);
  hipLaunchKernelGGL(k_order_blocks, dim3((unsigned)g.bh), dim3(kOrderThreads), 0, s, g, q_cnt,
                     order);
  return hipGetLastError();
}

template <bool kGen, int kR>
hipError_t launch_bwd_kernels(const Geo& g, const BwdArgs& a, const AttnGrid& ag,
                              hipStream_t s) {
  const dim3 grid((unsigned)ag.blocks), block(2 * kR);
  hipLaunchKernelGGL((k_attn_bwd_dq<kGen, kR>), grid, block, 0, s, g, a, ag);
  hipLaunchKernelGGL((k_attn_bwd_dkdv<kGen, kR>), grid, dim3(DkdvShape<kR>::kWaves * 64), 0, s,
                     g, a, ag);
  return hipGetLastError();
}

hipError_t launch_attention_bwd(const Geo& g, const BwdArgs& a, hipStream_t s) {
  const AttnGrid ag = attn_grid(g);
  const bool gen = g.ragged || g.L > 0;   // partial blocks or text blocks
  if (g.R == kSmallTile)
    return gen ? launch_bwd_kernels<true, kSmallTile>(g, a, ag, s)
               : launch_bwd_kernels<false, kSmallTile>(g, a, ag, s);
  return gen ? launch_bwd_kernels<true, kTileTokens>(g, a, ag, s)
             : launch_bwd_kernels<false, kTileTokens>(g, a, ag, s);
}

}  // namespace ssta

// Step 4 of SSTA: block-sparse attention over the kept (query block, key
// block) pairs ("HunyuanVideo 1.5 Technical Report" summary page, section
// "SSTA: Selective and Sliding Tile Attention", Step 4 and the attention
// equation): for each query token, softmax of scale*q.k over the tokens of
// the kept key blocks only, then the weighted sum of their values.
//
// gfx950 design.  One workgroup (4 waves) per query block of 128 tokens;
// each wave owns 32 queries (64-token blocks: two waves per 32 queries, each
// taking one 32-key half of every unit; see Blk).  The kernel computes the
// transposed scores
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = the
// wave's Q^T held in registers for the whole row), so each lane ends up with
// one query's scores for 64 of the 128 keys of a block and the row softmax
// needs a single cross-lane exchange (lane ^ 32).  The softmax runs online in
// fp32 in the log2 domain.  The probabilities never leave registers: the
// MFMA output layout of S^T is reused directly as the B operand of
// O^T += V^T P^T.  Each lane feeds key row kperm(lane) (bits 2 and 3 of the
// lane index swapped) into the S^T product, which makes every 8 output
// registers of a lane 8 consecutive keys, the A operand of the P.V product:
// channel d of 8 consecutive keys.  With token-major inputs V is gathered in
// token rows like K, and that operand comes from two transposing LDS reads
// (ds_read_b64_tr_b16) of 4 keys each; with dim-major V tiles it is one
// 16-byte read of a V^T row.  LDS rows carry a 16-byte-chunk XOR swizzle
// (K rows: chunk ^ row%16; V rows: chunk ^ 4*(row%4); V^T rows:
// chunk ^ (row/2)%8) so the MFMA operand reads are conflict-free.
// Schedule: the hardware deals workgroup ids round-robin over the 8 XCDs.
// The grid is laid out so that XCD x receives, head after head, the
// contiguous slice [x*c, (x+1)*c) of that head's query blocks (c = ceil(n/8))
// in a visiting order (block ids; 3D tiles of blocks for 64-token grids, see
// AttnGrid).
// All XCDs therefore work on the same one or two heads at any time, whose K
// and V (118 MB per head at the 720p 10 s shape) stay resident in the 256 MB
// MALL, while within an XCD neighbouring query blocks share most of their
// window blocks in that XCD's L2.  On a joint sequence the text query blocks,
// which run over every block, take the first workgroups of the grid, dealt
// over all XCDs, so they overlap the clip blocks instead of trailing them.
// Memory: each kept block is processed as two units of 64 keys.  A unit's K
// and V (16 KB each) go straight from global memory into LDS
// with buffer_load_dwordx4 ... lds (no register staging) into a two-slot
// ring; the next unit's loads are issued right after the barrier that frees
// its slot and overlap the whole current unit.  The buffer form (a per-head
// resource with a 32-bit offset, range-checked by the hardware) is used
// rather than global_load_lds because the compiler then tracks the LDS
// operand reads that follow with exact lgkmcnt waits instead of draining
// them all.  Kept-block ids are read 64 at a time into one register per lane
// and taken out with v_readlane, so no per-unit global load sits on the
// critical path.
// LDS operand reads are issued ahead of their products (up to 8 for K, the
// first 8 V operands before the softmax; with 64-token blocks from one asm
// block, see v_operands_tile), held in place by scheduling fences; waves
// raise their issue priority around the matrix-core sections.
// Softmax: the running max m is raised only when the probabilities formed
// with the current m would exceed 2^32 on some lane (always on a row's first
// unit), so most units need neither a max reduction nor an O rescale; the
// denominator is summed from the bf16-rounded probabilities with v_dot2 (the
// same weights the P.V product uses).
//
// Work per kept pair: 4*128^3 = 8.39 MFLOP on the matrix cores, 64 KB of
// K and V reads.  Bound: bf16 MFMA throughput (and the fp32 softmax that must
// overlap it).
#include "ssta_internal.h"

namespace ssta {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Blocks hold kR = 128 or 64 tokens; a workgroup has 4 waves and takes a key
// block in kR/64 units of 64 keys.  128-token blocks: each wave owns 32
// queries and every key of a unit.  64-token blocks (kSplit): the block's 64
// queries form two groups of 32, and each group is shared by two waves that
// take one 32-key half of every unit each, with their own running max and
// sums; the pair merges its two partial results at the end.  Both shapes
// thus run 4-wave workgroups, two per CU (64 KB of LDS each): two waves per
// SIMD.
template <int kR>
struct Blk {
  static constexpr int kWaves = 4;
  static constexpr bool kSplit = kR == 64;
  static constexpr int kTiles = kSplit ? 1 : 2;       // 32-key tiles of a unit per wave
  static constexpr int kLoads = 16 / kWaves;          // 1 KB loads per wave per 16 KB slot
  static constexpr int kUnits = kR / 64;              // 64-key units per block
  static constexpr int kBytes = kR * kHeadDim * 2;    // one block of one tensor
};
constexpr int kSlotBytes = 16384;                     // one unit of 64 keys: 16 KB of K or V
constexpr unsigned kWaitVm0 = 0x0F70;                    // s_waitcnt vmcnt(0)
// Scheduling fence that lets vector, scalar and transcendental ALU
// instructions move across it but keeps matrix, LDS and global memory
// instructions on their side, so LDS operand reads stay issued a fixed number
// of products ahead of their use.
// Largest per-lane probability sum of one unit accepted without raising the
// running max (see the softmax in the kernel).
constexpr float kMaxUnitSum = 4294967296.0f;   // 2^32
constexpr int kFenceKeepDs = 0x0002 | 0x0004 | 0x0400;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Token-row slots (64 rows of 256 B): 16-byte chunk c of row r sits at chunk
// c ^ row_swz(r).  K (read a whole 16-byte chunk per lane, 16 rows at a time):
// r % 16.  V (read 8 bytes per lane by the transposing loads, 4 rows at a
// time): 4 * (r % 4).  Both make the operand reads conflict-free.
template <bool kV>
__device__ __forceinline__ int row_swz(int row) {
  return kV ? 4 * (row & 3) : (row & 15);
}
__device__ __forceinline__ int swz_k(int row, int chunk) {
  return row * 256 + ((chunk ^ row_swz<false>(row)) << 4);
}
// V^T slot (128 channel rows of 128 B): chunk c of row d sits at chunk
// c ^ ((d / 2) % 8), so 16 consecutive rows read one chunk from 16 distinct
// bank groups.
__device__ __forceinline__ int swz_v(int d, int chunk) {
  return d * 128 + ((chunk ^ ((d >> 1) & 7)) << 4);
}

// A operand of O^T += V^T P^T for k-step (t, ks) and channel block db: lane
// (l32, hl) needs channel 32*db + l32 of the 8 keys 32t + 16ks + 8hl + (0..7).
// From a token-major V slot (rows of 256 B, swizzle row_swz<true>) this is two
// transposing reads (ds_read_b64_tr_b16): within each group of 16 lanes, lane
// j reads 4 channels of key j/4 of a 4-key row group, and lane i of the group
// receives channel i of those 4 keys.  v_lane_offset gives this lane's byte
// offset for channel block 0 and the first 4 keys of the hl half (the second
// 4 keys lie 1 KB further).  With row & 3 = j/4 the swizzle only flips the
// 64-byte group, bits 6-7 of the offset, which hold db ^ j/4: channel block db
// is at offset ^ (db << 6).
__device__ __forceinline__ int v_lane_offset(int lane) {
  const int j = lane & 15, grp = (lane >> 4) & 1, hl = lane >> 5;
  const int kq = j >> 2;                                   // key within the 4-row group
  const int chunk = 4 * kq + 2 * grp + ((j & 3) >> 1);     // swizzled 16-byte chunk, db = 0
  return (8 * hl + kq) * 256 + chunk * 16 + 8 * (j & 1);
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
template <bool kTok>
__device__ __forceinline__ bf16x8 v_operand(const uint8_t* sV, int t, int ks, int db, int l32,
                                            int hl, int vofs) {
  if (!kTok)
    return *reinterpret_cast<const bf16x8*>(sV + swz_v(32 * db + l32, 4 * t + 2 * ks + hl));
  const uint8_t* p = sV + (vofs ^ (db << 6)) + (32 * t + 16 * ks) * 256;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 1024));
  const auto w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, w);
}

// The 8 V operands of one 32-key tile t of a token-major V slot (operand i:
// ks = i/4, db = i%4, the addresses of v_operand), read by one asm block that
// waits for its own reads before it ends.  With the builtin the compiler,
// which cannot tell a transposing read's LDS address from the target of the
// next unit's direct loads, first waits for those loads to land (vmcnt(0));
// the slot read here is never a load target while it is read.  Used by the
// 64-token instance, whose waves run only 8 products between the unit's
// barrier and these reads, so the drain cost it 3% of its time; with 128-token
// blocks the same drain measured as free.
__device__ __forceinline__ void v_operands_tile(const uint8_t* sV, int t, int vofs, bf16x8* vr) {
  uint32_t b[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
    b[db] = (uint32_t)(uintptr_t)(const lds_u8*)(sV + (vofs ^ (db << 6)) + 32 * t * 256);
  long r[16];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:1024\n\t"
      "ds_read_b64_tr_b16 %2, %17\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:1024\n\t"
      "ds_read_b64_tr_b16 %4, %18\n\t"
      "ds_read_b64_tr_b16 %5, %18 offset:1024\n\t"
      "ds_read_b64_tr_b16 %6, %19\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:1024\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %9, %16 offset:5120\n\t"
      "ds_read_b64_tr_b16 %10, %17 offset:4096\n\t"
      "ds_read_b64_tr_b16 %11, %17 offset:5120\n\t"
      "ds_read_b64_tr_b16 %12, %18 offset:4096\n\t"
      "ds_read_b64_tr_b16 %13, %18 offset:5120\n\t"
      "ds_read_b64_tr_b16 %14, %19 offset:4096\n\t"
      "ds_read_b64_tr_b16 %15, %19 offset:5120\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
        "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
      : "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3])
      : "memory");
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const s16x4 lo = __builtin_bit_cast(s16x4, r[2 * i]);
    const s16x4 hi = __builtin_bit_cast(s16x4, r[2 * i + 1]);
    vr[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
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

// Direct global->LDS loads (buffer_load_dwordx4 ... lds).  A slot is 16 KB:
// each wave issues kLoads instructions of 1 KB; lane i of an instruction lands
// at byte 16*i of its 1 KB destination block, so the source address of each
// lane is chosen to put the right (swizzled) chunk there.  The per-lane byte
// offsets depend only on the lane and wave (computed once); the unit base is
// uniform, so the loads use a scalar base plus a 32-bit lane offset.
template <int kR>
struct DmaOffsets {
  uint32_t k[Blk<kR>::kLoads], v[Blk<kR>::kLoads];
};

// kTok: K and V are read from token-major [.., S, 128] memory, so key row r
// of a unit comes from token in_block_offset(r) of its block (a 256-byte
// row); V rows land like K rows, with their own swizzle.  Otherwise K comes
// from tile-major blocks and V^T from dim-major tiles whose channel rows hold
// 2*kR bytes.
template <bool kTok, int kR>
__device__ __forceinline__ DmaOffsets<kR> dma_offsets(const Geo& g, int wave, int lane) {
  DmaOffsets<kR> o;
#pragma unroll
  for (int mm = 0; mm < Blk<kR>::kLoads; ++mm) {
    const int b = Blk<kR>::kLoads * wave + mm;   // 1 KB destination block
    const int row = 4 * b + (lane >> 4);         // token rows 4b .. 4b+3
    const uint32_t src_row = kTok ? in_block_offset(g, row) : (uint32_t)row;
    o.k[mm] = src_row * 256 + (((lane & 15) ^ row_swz<false>(row)) << 4);
    if (kTok) {
      o.v[mm] = src_row * 256 + (((lane & 15) ^ row_swz<true>(row)) << 4);
    } else {
      const int d = 8 * b + (lane >> 3);         // V^T: channel rows 8b .. 8b+7
      o.v[mm] = d * (2 * kR) + (((lane & 7) ^ ((d >> 1) & 7)) << 4);
    }
  }
  return o;
}

// Buffer resource over one head's K, K_t or V_t (bytes; n_rows blocks);
// loads beyond num_records return zero instead of touching other memory.
template <int kR>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint8_t* base, int64_t n_rows) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0,
                                           (int)(n_rows * Blk<kR>::kBytes), 0x00020000);
}

// Half p (keys 64p .. 64p+63) of the K (kV: V) block j, as 64 token rows.
// Tile-major: 64 contiguous rows.  Token-major: the rows of the block's
// tokens; in-block positions are a bit-field code of (t, y, x) offsets, so
// position 64p + r lies at token offset in_block_offset(64p) +
// in_block_offset(r) from the block's origin.  Blocks from n_tiles on are
// text blocks, whose positions are consecutive tokens after the clip's.
// kGen (ragged grids, joint text): bit r of `valid` says whether position
// 64p + r of the block exists.  In a unit with missing positions the scalar
// base is the block's first token, which every block has, and a missing row
// reads that row (both K and V: a missing key's probability is exactly zero,
// and the row it reads is a finite row of the same head).  The scalar offset
// is outside the buffer range check, so no base may point past the head's
// tokens.  `offs`: the K or V offsets of a DmaOffsets<kR>.
template <bool kTokK, bool kGen, int kR, bool kV>
__device__ __forceinline__ void dma_rows(uint8_t* dst, __amdgpu_buffer_rsrc_t rs, const Geo& g,
                                         int64_t j, int p, int wave, int lane, uint64_t valid,
                                         const uint32_t* offs) {
  constexpr int kL = Blk<kR>::kLoads;
  const bool text = kGen && kTokK && j >= g.n_tiles;
  const bool part = kGen && kTokK && valid != ~0ull;
  uint32_t so, half = 0u;
  if (kTokK) {
    const uint32_t origin =
        text ? (uint32_t)(g.N + (j - g.n_tiles) * kR) : block_origin32(g, (uint32_t)j);
    half = p ? (text ? 64u : in_block_offset(g, 64)) * 256u : 0u;
    so = origin * 256u + (part ? 0u : half);
  } else {
    so = (uint32_t)(j * Blk<kR>::kBytes + p * kSlotBytes);
  }
#pragma unroll
  for (int mm = 0; mm < kL; ++mm) {
    uint32_t vo = offs[mm];
    const int r = 4 * (kL * wave + mm) + (lane >> 4);
    if (text) vo = r * 256 + (((lane & 15) ^ row_swz<kV>(r)) << 4);
    if (part) vo = ((valid >> r) & 1u) ? vo + half : (vo & 255u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_u8*)(dst + (kL * wave + mm) * 1024), 16,
                                             vo, so, 0, 0);
  }
}

// Unit p of block j from token-major K and V.  The common case, a clip
// block whose unit has every position, takes one straight path shared with
// the instance without partial blocks (one uniform test), so its set-up stays
// short between the barrier and the unit's products; text blocks and units
// with missing positions take the general path of dma_rows.
template <bool kGen, int kR>
__device__ __forceinline__ void dma_unit_tok(uint8_t* dk, uint8_t* dv, __amdgpu_buffer_rsrc_t krs,
                                             __amdgpu_buffer_rsrc_t vrs, const Geo& g, int64_t j,
                                             int p, int wave, int lane, uint64_t valid,
                                             const uint32_t* ok, const uint32_t* ov) {
  constexpr int kL = Blk<kR>::kLoads;
  if (!kGen || (j < g.n_tiles && valid == ~0ull)) {
    const uint32_t so =
        block_origin32(g, (uint32_t)j) * 256u + (p ? in_block_offset(g, 64) * 256u : 0u);
#pragma unroll
    for (int mm = 0; mm < kL; ++mm)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_u8*)(dk + (kL * wave + mm) * 1024), 16,
                                               ok[mm], so, 0, 0);
#pragma unroll
    for (int mm = 0; mm < kL; ++mm)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_u8*)(dv + (kL * wave + mm) * 1024), 16,
                                               ov[mm], so, 0, 0);
    return;
  }
  dma_rows<true, kGen, kR, false>(dk, krs, g, j, p, wave, lane, valid, ok);
  dma_rows<true, kGen, kR, true>(dv, vrs, g, j, p, wave, lane, valid, ov);
}

// Which of positions 64p .. 64p+63 of block j exist: all of them unless the
// block is an edge block of a ragged grid or the last, partial text block.
template <bool kGen, int kR>
__device__ __forceinline__ uint64_t unit_valid(const Geo& g, int64_t j, int p, int lane) {
  if (!kGen) return ~0ull;
  if (j >= g.n_tiles) {
    const int64_t u0 = (j - g.n_tiles) * kR + 64 * p;   // first text token
    if (u0 + 64 <= g.L) return ~0ull;
    return __ballot(u0 + lane < g.L);
  }
  if (!g.ragged) return ~0ull;
  const BlockExtent e = block_extent(g, (uint32_t)j);
  if (e.full) return ~0ull;
  return __ballot(pos_exists(g, e, 64 * p + lane));
}
// Unit p of V^T block j: bytes 128p .. 128p+127 of each channel row (offv:
// the V^T offsets of a DmaOffsets<kR>).
template <int kR>
__device__ __forceinline__ void dma_v(uint8_t* dst, __amdgpu_buffer_rsrc_t rs, int64_t j, int p,
                                      int wave, const uint32_t* offv) {
  constexpr int kL = Blk<kR>::kLoads;
  const uint32_t so = (uint32_t)(j * Blk<kR>::kBytes + p * 128);
#pragma unroll
  for (int mm = 0; mm < kL; ++mm)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_u8*)(dst + (kL * wave + mm) * 1024), 16,
                                             offv[mm], so, 0, 0);
}

// kTok: Q, K, V and O are token-major [B, h, S, 128] (the query block is
// gathered, the key blocks are gathered by the LDS loads and the output is
// scattered directly); otherwise Q, K and O are tile-major
// [B, h, n_rows, R, 128] and V is dim-major tiles [B, h, n_rows, 128, R].
// kGen: the instance for ragged grids and joint text (masked partial blocks,
// text blocks always kept, text query blocks dense); grids the block size
// divides, without text, run the other instance.
// kR: tokens per block (128: two units per key block; 64: one unit, its two
// halves taken by two waves per query group, see Blk).
template <bool kTok, bool kGen, int kR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void k_attn_fwd(Geo g, AttnArgs a, AttnGrid grid) {
  // K slots at 0 and 16 KB, V (or V^T) slots at 32 and 48 KB.
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * kSlotBytes];

  // Text query blocks first, then head-synchronous XCD slices of the clip
  // blocks (see the file comment and attn_grid).
  int64_t bh, qi;
  if (!attn_block<kGen>(g, grid, blockIdx.x, bh, qi)) return;
  const int64_t row = bh * g.n_rows + qi;        // LSE and tile-major rows
  const bool qtext = kGen && qi >= g.n_tiles;    // a text query block

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int kperm = (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  constexpr int64_t kTileElems = kR * kHeadDim;
  constexpr int kUnits = Blk<kR>::kUnits;
  constexpr bool kSplit = Blk<kR>::kSplit;
  constexpr int kT = Blk<kR>::kTiles;
  // query group (32 queries) and, with split units, the 32-key half of each
  // unit this wave takes
  const int qg = kSplit ? (wave & 1) : wave;
  const int kh = kSplit ? (wave >> 1) : 0;
  // unit tile tt of this wave is the unit's keys 32 * tile(tt) .. + 31
  auto tile = [&](int tt) { return kSplit ? kh : tt; };

  // qb: this lane's query row is qb + (kTok ? 0 : qrow * 128).  A query
  // position its block lacks (ragged edge, past the text) reads the block's
  // first token instead; its output is not written.
  const int qrow = qg * 32 + l32;
  const bool qvalid =
      (unit_valid<kGen, kR>(g, qi, qg >> 1, lane) >> (32 * (qg & 1) + l32)) & 1u;
  // token of the query within its head (clip tokens first, then the text)
  const int64_t qtok =
      qtext ? g.N + (qi - g.n_tiles) * kR + (qvalid ? qrow : 0)
            : block_first_token(g, (uint32_t)qi) + (qvalid ? in_block_offset(g, qrow) : 0u);
  const uint16_t* qb = static_cast<const uint16_t*>(a.q_t) + row * kTileElems;
  // S tokens of each earlier head precede this one in token-major tensors
  if (kTok) qb = static_cast<const uint16_t*>(a.q_t) + (bh * g.S + qtok) * kHeadDim;
  // K: token-major (S rows per head) or tile-major (n_rows blocks per head)
  const uint8_t* kb = reinterpret_cast<const uint8_t*>(
      static_cast<const uint16_t*>(a.k_t) + bh * (kTok ? g.S * kHeadDim : g.n_rows * kTileElems));
  // V: token-major like K, or dim-major tiles
  const uint8_t* vb = reinterpret_cast<const uint8_t*>(
      static_cast<const uint16_t*>(a.v_t) + bh * (kTok ? g.S * kHeadDim : g.n_rows * kTileElems));
  // The row's key blocks: the kept list (clip rows), then every text block;
  // a text query block, or dense attention, takes every block in order.
  const bool all_blocks = a.kv_cnt == nullptr || qtext;
  const int64_t kvrow = bh * g.n_tiles + qi;
  // Lists come from the caller: the count is clamped to the row's capacity
  // and every id to a clip block, so a malformed list reads only the head's
  // own blocks.
  const int listed = all_blocks ? 0 : min(max(a.kv_cnt[kvrow], 0), a.max_kept);
  const int cnt = all_blocks ? (int)g.n_rows : listed + (kGen ? g.n_txt : 0);
  const int32_t* idx = all_blocks ? nullptr : a.kv_idx + kvrow * a.max_kept;

  // B operand of S^T = K Q^T: query (32*wave + l32), channels 16*s + 8*hl .. +8.
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

  // Unit u = keys 64*(u%kUnits) .. of the (u/kUnits)-th kept block, in slot
  // u%2 of the K and V rings; unit u+1 is loaded while unit u is computed.
  const int units = kUnits * cnt;
  const DmaOffsets<kR> doff = dma_offsets<kTok, kR>(g, wv, lane);
  // token-major K spans S rows of 256 B; tiles span n_rows x 32 KB
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kb), (short)0,
                                        (int)(kTok ? g.S * 256 : g.n_rows * Blk<kR>::kBytes),
                                        0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      kTok ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vb), (short)0, (int)(g.S * 256),
                                               0x00020000)
           : head_rsrc<kR>(vb, g.n_rows);
  // V operand reads: this lane's byte offset within a token-major V slot
  // (see v_operand)
  const int vofs = kTok ? v_lane_offset(lane) : 0;
  // Kept-block ids, 64 at a time: lane i holds entry ibase + i.
  int ibase = 0;
  const int last_tile = (int)g.n_tiles - 1;
  int ids = (!all_blocks && lane < listed) ? idx[lane] : 0;
  // On a ragged grid, which of the 64 entries are whole blocks (one vector
  // test per 64 entries instead of a scalar one per unit).
  auto whole = [&]() -> uint64_t {
    if (!kGen || all_blocks || !g.ragged) return 0ull;
    const uint32_t j = (uint32_t)min(max(ids, 0), last_tile);
    return __ballot(ibase + lane < listed && block_extent(g, j).full);
  };
  uint64_t whole_m = whole();
  auto block_at = [&](int pos) -> int64_t {
    if (all_blocks) return pos;
    if (kGen && pos >= listed) return g.n_tiles + (pos - listed);   // a text block
    if (pos >= ibase + 64) {   // uniform: next 64 entries
      ibase += 64;
      ids = (ibase + lane < listed) ? idx[ibase + lane] : 0;
      whole_m = whole();
    }
    return min(max(__builtin_amdgcn_readlane(ids, pos - ibase), 0), last_tile);
  };
  // positions of unit p of the block at list position pos (after block_at)
  auto valid_at = [&](int pos, int64_t j, int p) -> uint64_t {
    if (kGen && !all_blocks && pos < listed && ((whole_m >> (pos - ibase)) & 1u)) return ~0ull;
    return unit_valid<kGen, kR>(g, j, p, lane);
  };
  uint64_t valid_next = ~0ull;   // positions of the unit loaded last that exist
  if (units > 0) {
    const int64_t j = block_at(0);
    valid_next = valid_at(0, j, 0);
    if (kTok) {
      dma_unit_tok<kGen, kR>(smem, smem + 2 * kSlotBytes, krs, vrs, g, j, 0, wv, lane,
                             valid_next, doff.k, doff.v);
    } else {
      dma_rows<kTok, kGen, kR, false>(smem, krs, g, j, 0, wv, lane, valid_next, doff.k);
      dma_v<kR>(smem + 2 * kSlotBytes, vrs, j, 0, wv, doff.v);
    }
  }

  for (int u = 0; u < units; ++u) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);   // this wave's loads of unit u have landed
    __syncthreads();                        // ... every wave's; and unit u-1 is done
    const int slot = u & 1;
    const uint64_t valid = valid_next;
    if (u + 1 < units) {
      const int64_t j = block_at((u + 1) / kUnits);
      const int p = (u + 1) % kUnits;
      valid_next = valid_at((u + 1) / kUnits, j, p);
      if (kTok) {
        dma_unit_tok<kGen, kR>(smem + (1 - slot) * kSlotBytes, smem + (3 - slot) * kSlotBytes,
                               krs, vrs, g, j, p, wv, lane, valid_next, doff.k, doff.v);
      } else {
        dma_rows<kTok, kGen, kR, false>(smem + (1 - slot) * kSlotBytes, krs, g, j, p, wv, lane,
                                        valid_next, doff.k);
        dma_v<kR>(smem + (3 - slot) * kSlotBytes, vrs, j, p, wv, doff.v);
      }
    }
    const uint8_t* sK = smem + slot * kSlotBytes;
    const uint8_t* sV = smem + (2 + slot) * kSlotBytes;

    // S^T: 8 * kT products in the order (st, tt); their K operands are read
    // kKAhead products ahead so the LDS latency overlaps the matrix cores.
    // The A operand row of lane l32 is key kperm(l32), so output register r
    // of lane (l32, hl) of s[tt] holds query l32 and key
    // 32*tile(tt) + 16*(r/8) + 8*hl + r%8: each group of 8 registers is 8
    // consecutive keys.
    constexpr int kKAhead = 8;
    constexpr int kSProducts = 8 * kT;
    __builtin_amdgcn_s_setprio(1);
    f32x16 s[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = 0.0f;
    bf16x8 kr[kKAhead];
#pragma unroll
    for (int i = 0; i < kKAhead; ++i)
      kr[i] = *reinterpret_cast<const bf16x8*>(
          sK + swz_k(32 * tile(i % kT) + kperm, 2 * (i / kT) + hl));
#pragma unroll
    for (int i = 0; i < kSProducts; ++i) {
      const int st = i / kT, tt = i % kT;
      s[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[i % kKAhead], qf[st], s[tt], 0, 0, 0);
      const int n = i + kKAhead;
      if (n < kSProducts)
        kr[i % kKAhead] = *reinterpret_cast<const bf16x8*>(
            sK + swz_k(32 * tile(n % kT) + kperm, 2 * (n / kT) + hl));
      __builtin_amdgcn_sched_barrier(0);
    }
    // Keys an edge block of a ragged grid lacks get a score far below any
    // real one, so their probabilities vanish (position 0 always exists, so
    // a row's first unit has a real key; a wave's second half of a unit may
    // have none, which the softmax below handles).
    if (kGen && valid != ~0ull) {
      const uint64_t vl = valid >> (8 * hl);
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((vl >> (32 * tile(t) + 16 * (r >> 3) + (r & 7))) & 1u)) s[t][r] = -1.0e30f;
    }

    // V operands of the first kVAhead P.V products (order (tt, ks, db)),
    // requested before the softmax so they arrive while it runs.
    constexpr int kVAhead = 8;
    constexpr int kVProducts = 8 * kT;
    bf16x8 vr[kVAhead];
    if (kTok && kSplit) {
      v_operands_tile(sV, tile(0), vofs, vr);
    } else {
#pragma unroll
      for (int i = 0; i < kVAhead; ++i)
        vr[i] = v_operand<kTok>(sV, tile(i >> 3), (i >> 2) & 1, i & 3, l32, hl, vofs);
    }

    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(kFenceKeepDs);

    // Online softmax in the log2 domain against the running max m, which is
    // only raised when needed: the probabilities are first formed with the
    // current m; if some lane's sum over its 32 keys leaves [0, 2^32] (always
    // on a row's first unit, where m = -inf), the unit's max is taken, O and l
    // are rescaled and the probabilities are formed again.  Every probability
    // that enters O is therefore at most 2^32.
    // P^T as B operand of k-step (t, ks): registers 8*ks .. 8*ks+7, which are
    // keys 32*t + 16*ks + 8*hl + (0..7) of the unit.  The denominator sums the
    // bf16-rounded probabilities (the weights the P.V product uses) with v_dot2.
    bf16x8 pf[kT][2];
    float lu;
    auto probabilities = [&]() {
      float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
      for (int t = 0; t < kT; ++t)
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
      lu = l0 + l1;
    };
    probabilities();
    if (__any(!(lu <= kMaxUnitSum))) {
      float x0 = max3f(s[0][0], s[0][1], s[0][2]);
      float x1 = max3f(s[kT - 1][0], s[kT - 1][1], s[kT - 1][2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) {
        x0 = max3f(x0, s[0][r], s[0][r + 1]);
        x1 = max3f(x1, s[kT - 1][r], s[kT - 1][r + 1]);
      }
      const float mx = pair_max(max3f(max3f(x0, x1, s[0][15]), s[kT - 1][15], -INFINITY)) * c;
      float m_new = fmaxf(m, mx);
      // With split units a wave's half of a unit can lack every key (scores
      // -1e30): a floor halfway to that score keeps such keys' probabilities
      // at 0 before the wave has seen a real key.  Any real score lies above
      // it, so the floor never changes a real running max.
      if (kSplit) m_new = fmaxf(m_new, -5.0e29f * c);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m = m_new;
      probabilities();
    }
    l += lu;

    __builtin_amdgcn_s_setprio(1);
    // O^T += V^T P^T in the order (t, ks, db); A operand: channel d of the
    // same 8 consecutive keys 32t + 16ks + 8hl + (0..7) (see v_operand).
#pragma unroll
    for (int i = 0; i < kVProducts; ++i) {
      const int tt = i >> 3, ks = (i >> 2) & 1, db = i & 3;
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[i % kVAhead], pf[tt][ks], o[db], 0, 0, 0);
      const int n = i + kVAhead;
      if (n < kVProducts)
        vr[i % kVAhead] = v_operand<kTok>(sV, tile(n >> 3), (n >> 2) & 1, n & 3, l32, hl, vofs);
      __builtin_amdgcn_sched_barrier(kFenceKeepDs);
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // Epilogue: lane holds query qrow, channels 32*db + 8*g4 + 4*hl + (0..3).
  // A query position its block lacks has no output row (token order) or a
  // zero row (tile order), and LSE -inf.
  float lt = pair_sum(l);
  if (kSplit) {
    // The second wave of each query group hands its running max, sum and O
    // to the first through LDS (the ring is free: every wave is past its
    // last unit and no load is in flight); the first rescales both to the
    // larger max and adds them.
    float* xs = reinterpret_cast<float*>(smem) + qg * (66 * 64);
    __syncthreads();
    if (kh == 1) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xs[(16 * db + r) * 64 + lane] = o[db][r];
      xs[64 * 64 + lane] = m;
      xs[65 * 64 + lane] = lt;
    }
    __syncthreads();
    if (kh == 1) return;
    const float m2 = xs[64 * 64 + lane], lt2 = xs[65 * 64 + lane];
    const float mt = fmaxf(m, m2);
    // a side without keys has m = -inf and contributes nothing; if both
    // have none, lt stays 0 (the row's output is 0, its LSE -inf)
    const float a1 = mt == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mt);
    const float a2 = mt == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m2 - mt);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * a1 + xs[(16 * db + r) * 64 + lane] * a2;
    lt = lt * a1 + lt2 * a2;
    m = mt;
  }
  const float inv = (lt > 0.0f && qvalid) ? 1.0f / lt : 0.0f;
  uint16_t* ob = static_cast<uint16_t*>(a.o_t) + row * kTileElems + qrow * kHeadDim;
  if (kTok) ob = static_cast<uint16_t*>(a.o_t) + (bh * g.S + qtok) * kHeadDim;
  if (!kTok || qvalid) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (!kGen || qvalid) ? (__bf16)(o[db][4 * g4 + e] * inv) : (__bf16)0.0f;
        *reinterpret_cast<bf16x4*>(ob + 32 * db + 8 * g4 + 4 * hl) = w;
      }
  }
  if (a.lse != nullptr && hl == 0) {
    const float v =
        (lt > 0.0f && qvalid) ? (m + __log2f(lt)) * 0.69314718055994530942f : -INFINITY;
    a.lse[row * kR + qrow] = v;
  }
}

}  // namespace

hipError_t launch_attention(const Geo& g, const AttnArgs& a, hipStream_t s) {
  const AttnGrid ag = attn_grid(g);
  const int64_t blocks = ag.blocks;
  // grids the block size divides, without text, take the instance without
  // partial-block masking and text blocks
  const bool gen = g.ragged || g.L > 0;
  const dim3 grid((unsigned)blocks);
  if (g.R == kSmallTile) {
    const dim3 block(256);
    if (a.token_io && gen)
      hipLaunchKernelGGL((k_attn_fwd<true, true, kSmallTile>), grid, block, 0, s, g, a, ag);
    else if (a.token_io)
      hipLaunchKernelGGL((k_attn_fwd<true, false, kSmallTile>), grid, block, 0, s, g, a, ag);
    else if (gen)
      hipLaunchKernelGGL((k_attn_fwd<false, true, kSmallTile>), grid, block, 0, s, g, a, ag);
    else
      hipLaunchKernelGGL((k_attn_fwd<false, false, kSmallTile>), grid, block, 0, s, g, a, ag);
  } else {
    const dim3 block(256);
    if (a.token_io && gen)
      hipLaunchKernelGGL((k_attn_fwd<true, true, kTileTokens>), grid, block, 0, s, g, a, ag);
    else if (a.token_io)
      hipLaunchKernelGGL((k_attn_fwd<true, false, kTileTokens>), grid, block, 0, s, g, a, ag);
    else if (gen)
      hipLaunchKernelGGL((k_attn_fwd<false, true, kTileTokens>), grid, block, 0, s, g, a, ag);
    else
      hipLaunchKernelGGL((k_attn_fwd<false, false, kTileTokens>), grid, block, 0, s, g, a, ag);
  }
  return hipGetLastError();
}

}  // namespace ssta

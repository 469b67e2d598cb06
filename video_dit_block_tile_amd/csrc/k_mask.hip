// Steps 3 and 4 of SSTA up to the attention call: the sliding-tile window
// (Step 3, M_sta) combined with the selected blocks (Step 4) into compacted
// kept-block lists ("HunyuanVideo 1.5 Technical Report" summary page, section
// "SSTA: Selective and Sliding Tile Attention").
//
// One thread per query-block row.  The window is enumerated from the block's
// coordinates in ascending block id (t, then y, then x), clipped at the grid
// edge, and merged with the row's ascending top-k ids, so the list comes out
// ascending and duplicate-free without sorting.  Union by default; with
// combine_and only blocks in both.  Integer work; the kernel writes about
// 4*(max_kept+1) bytes per row and is bound by launch latency at the shapes
// used here.
#include "ssta_internal.h"

namespace ssta {
namespace {

struct RowWriter {
  int32_t* idx;
  int32_t cap;
  int32_t cnt;
  uint32_t* bm;        // nullable
  int64_t words;
  int64_t cur_word;
  uint32_t acc;

  __device__ void emit(int32_t j) {
    if (cnt < cap) idx[cnt] = j;
    ++cnt;
    if (bm != nullptr) {
      const int64_t w = j >> 5;
      while (cur_word < w) {
        bm[cur_word++] = acc;
        acc = 0u;
      }
      acc |= 1u << (j & 31);
    }
  }
  __device__ void finish() {
    for (int32_t p = cnt; p < cap; ++p) idx[p] = -1;
    if (bm != nullptr) {
      while (cur_word < words) {
        bm[cur_word++] = acc;
        acc = 0u;
      }
    }
  }
};

__global__ __launch_bounds__(256) void k_build_mask(Geo g, MaskArgs a) {
  const int64_t rows = g.bh * g.n_tiles;
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  const int64_t n = g.n_tiles;
  const int64_t i = row % n;
  const int ti = (int)(i / ((int64_t)g.ny * g.nx)), yi = (int)((i / g.nx) % g.ny),
            xi = (int)(i % g.nx);
  const int t0 = max(ti - a.wt, 0), t1 = min(ti + a.wt, g.nt - 1);
  const int y0 = max(yi - a.wh, 0), y1 = min(yi + a.wh, g.ny - 1);
  const int x0 = max(xi - a.ww, 0), x1 = min(xi + a.ww, g.nx - 1);
  const int32_t* tk = a.topk_idx + row * a.k_width;
  const int kw = a.k_width;

  RowWriter w;
  w.idx = a.kv_idx + row * a.max_kept;
  w.cap = a.max_kept;
  w.cnt = 0;
  w.bm = a.bitmask != nullptr ? a.bitmask + row * ((n + 31) / 32) : nullptr;
  w.words = (n + 31) / 32;
  w.cur_word = 0;
  w.acc = 0u;

  int p = 0;
  for (int t = t0; t <= t1; ++t)
    for (int y = y0; y <= y1; ++y)
      for (int x = x0; x <= x1; ++x) {
        const int32_t wj = (int32_t)(((int64_t)t * g.ny + y) * g.nx + x);
        while (p < kw && tk[p] >= 0 && tk[p] < wj) {
          if (!a.combine_and) w.emit(tk[p]);
          ++p;
        }
        if (p < kw && tk[p] == wj) {
          w.emit(wj);
          ++p;
        } else if (!a.combine_and) {
          w.emit(wj);
        }
      }
  while (p < kw && tk[p] >= 0) {
    if (!a.combine_and) w.emit(tk[p]);
    ++p;
  }
  w.finish();
  a.kv_cnt[row] = min(w.cnt, w.cap);
}

}  // namespace

hipError_t launch_build_mask(const Geo& g, const MaskArgs& a, hipStream_t s) {
  const int64_t rows = g.bh * g.n_tiles;
  hipLaunchKernelGGL(k_build_mask, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, g, a);
  return hipGetLastError();
}

}  // namespace ssta

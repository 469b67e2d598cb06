// Measurement aid, not a step of the method: back-to-back bf16 matrix-core
// products (v_mfma_f32_32x32x16_bf16) on register-resident operands, so the
// sustained matrix rate and clock of the chip can be measured next to the
// attention kernel.  Each wave runs four independent accumulation chains on
// operands it reads once; the data the products see (random or constant)
// decides how much power they draw.
#include "ssta_internal.h"

namespace ssta {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void k_calibrate_mfma(const bf16x8* operands, float* sink,
                                                         int iters) {
  const int lane = threadIdx.x & 63;
  const bf16x8 a0 = operands[lane], a1 = operands[64 + lane];
  const bf16x8 b0 = operands[128 + lane], b1 = operands[192 + lane];
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_calibrate_mfma(const void* operands, float* sink, int grid, int iters,
                                 hipStream_t s) {
  hipLaunchKernelGGL(k_calibrate_mfma, dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const bf16x8*>(operands), sink, iters);
  return hipGetLastError();
}

}  // namespace ssta

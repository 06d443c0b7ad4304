// Combine ("DeepSeek-V3.2-Exp · Mixture of experts", MoE.forward excerpt): an fp32
// accumulator per token; the routed experts' rows, each times its routing weight, are
// added in ascending expert order, then the shared expert's row; the sum is returned in
// x's dtype. Every multiply and add rounds to fp32 separately (no fused multiply-add),
// so the order of operations is the loop's.
//
// Also the per-token 1x128 activation quantisation for fp8 blocks.
#include <math.h>

#include <algorithm>

#include "combine_dev.h"

namespace moe {

template <bool kBf16>
__global__ __launch_bounds__(CT) void combine(const int32_t* __restrict__ idx, const float* __restrict__ w,
                                              const int32_t* __restrict__ row_of, const void* __restrict__ o_routed,
                                              const void* __restrict__ o_shared, void* __restrict__ out, int K,
                                              int D) {
  __shared__ int srow[kMaxTopK];
  __shared__ float sw[kMaxTopK];
  combine_token<kBf16, CT>(blockIdx.x, blockIdx.y, gridDim.y, srow, sw, idx, w, row_of, o_routed, o_shared, out, K, D);
}

// 16 lanes per (token, 128 columns), 8 values each: scale = amax / 448 (1 when amax = 0),
// codes = e4m3(x / scale).
__global__ __launch_bounds__(256) void act_quant(const bf16_t* __restrict__ x, uint8_t* __restrict__ xq,
                                                 float* __restrict__ sx, int64_t nblocks) {
#pragma clang fp contract(off)
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = g >> 4;
  const int l16 = threadIdx.x & 15;
  if (blk >= nblocks) return;  // whole 16-lane groups leave together
  const i32x4 v = ld16(x + blk * 128 + l16 * 8);
  float f[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t p = (uint32_t)v[j];
    f[2 * j] = bf16_to_f32((bf16_t)(p & 0xFFFF));
    f[2 * j + 1] = bf16_to_f32((bf16_t)(p >> 16));
  }
  float am = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(f[j]));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  const float scale = am > 0.f ? am / 448.0f : 1.0f;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    lo |= (f32x2_to_e4m3(f[2 * j] / scale, f[2 * j + 1] / scale) & 0xFFFFu) << (16 * j);
    hi |= (f32x2_to_e4m3(f[4 + 2 * j] / scale, f[5 + 2 * j] / scale) & 0xFFFFu) << (16 * j);
  }
  *reinterpret_cast<uint2*>(xq + blk * 128 + l16 * 8) = make_uint2(lo, hi);
  if (l16 == 0) sx[blk] = scale;
}

hipError_t launch_combine(const Dims& d, const int32_t* idx, const float* w, const int32_t* row_of,
                          const void* o_routed, const void* o_shared, void* out, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  // split the columns over more blocks when there are few tokens
  const unsigned ysplit = d.T >= 1024 ? 1u : (unsigned)std::max(1, std::min(8, d.D / (CT * 8)));
  if (d.dtype == 0)
    MOE_LAUNCH(combine<false>, dim3((unsigned)d.T, ysplit), dim3(CT), 0, s, idx, w, row_of, o_routed, o_shared,
               out, d.K, d.D);
  else
    MOE_LAUNCH(combine<true>, dim3((unsigned)d.T, ysplit), dim3(CT), 0, s, idx, w, row_of, o_routed, o_shared,
               out, d.K, d.D);
  return hipGetLastError();
}

hipError_t launch_act_quant(const Dims& d, const bf16_t* x, uint8_t* xq, float* sx, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  int64_t nb = d.T * (d.D / 128);
  MOE_LAUNCH(act_quant, dim3((unsigned)((nb + 15) / 16)), dim3(256), 0, s, x, xq, sx, nb);
  return hipGetLastError();
}

}  // namespace moe

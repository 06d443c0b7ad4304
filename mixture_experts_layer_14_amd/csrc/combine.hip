// Combine ("DeepSeek-V3.2-Exp · Mixture of experts", MoE.forward excerpt): an fp32
// accumulator per token; the routed experts' rows, each times its routing weight, are
// added in ascending expert order, then the shared expert's row; the sum is returned in
// x's dtype. Every multiply and add rounds to fp32 separately (no fused multiply-add),
// so the order of operations is the loop's.
//
// Also the per-token 1x128 activation quantisation for fp8 blocks.
#include <math.h>

#include <algorithm>

#include "kernels.h"

namespace moe {

constexpr int kMaxTopK = 16;

// One block per token. The token's (expert, weight, row) triples are sorted by expert.
template <bool kBf16>
__global__ __launch_bounds__(256) void combine(const int32_t* __restrict__ idx, const float* __restrict__ w,
                                               const int32_t* __restrict__ row_of, const void* __restrict__ o_routed,
                                               const void* __restrict__ o_shared, void* __restrict__ out, int K,
                                               int D) {
#pragma clang fp contract(off)
  __shared__ int srow[kMaxTopK];
  __shared__ float sw[kMaxTopK];
  const int t = blockIdx.x;
  if (threadIdx.x == 0) {
    int ek[kMaxTopK], rk[kMaxTopK];
    float wk[kMaxTopK];
    for (int k = 0; k < K; ++k) {
      int e = idx[(size_t)t * K + k], r = row_of[(size_t)t * K + k];
      float v = w[(size_t)t * K + k];
      int j = k;
      while (j > 0 && ek[j - 1] > e) {
        ek[j] = ek[j - 1];
        rk[j] = rk[j - 1];
        wk[j] = wk[j - 1];
        --j;
      }
      ek[j] = e;
      rk[j] = r;
      wk[j] = v;
    }
    for (int k = 0; k < K; ++k) {
      srow[k] = rk[k];
      sw[k] = wk[k];
    }
  }
  __syncthreads();
  if (kBf16) {
    const bf16_t* O = static_cast<const bf16_t*>(o_routed);
    const bf16_t* SH = static_cast<const bf16_t*>(o_shared) + (size_t)t * D;
    bf16_t* Y = static_cast<bf16_t*>(out) + (size_t)t * D;
    for (int c = (blockIdx.y * 256 + threadIdx.x) * 8; c < D; c += gridDim.y * 256 * 8) {
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = 0.f;
      // all rows are loaded before the in-order accumulation
      i32x4 rows[kMaxTopK];
#pragma unroll
      for (int k = 0; k < kMaxTopK; ++k)
        if (k < K) rows[k] = ld16(O + (size_t)srow[k] * D + c);
      i32x4 v = ld16(SH + c);
#pragma unroll
      for (int k = 0; k < kMaxTopK; ++k) {
        if (k >= K) continue;
        const float wk = sw[k];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t p = (uint32_t)rows[k][j];
          y[2 * j] = y[2 * j] + bf16_to_f32((bf16_t)(p & 0xFFFF)) * wk;
          y[2 * j + 1] = y[2 * j + 1] + bf16_to_f32((bf16_t)(p >> 16)) * wk;
        }
      }
      i32x4 res;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t p = (uint32_t)v[j];
        float a = y[2 * j] + bf16_to_f32((bf16_t)(p & 0xFFFF));
        float b = y[2 * j + 1] + bf16_to_f32((bf16_t)(p >> 16));
        res[j] = (int)pack_bf16x2(a, b);
      }
      *reinterpret_cast<i32x4*>(Y + c) = res;
    }
  } else {
    const float* O = static_cast<const float*>(o_routed);
    const float* SH = static_cast<const float*>(o_shared) + (size_t)t * D;
    float* Y = static_cast<float*>(out) + (size_t)t * D;
    for (int c = blockIdx.y * 256 + threadIdx.x; c < D; c += gridDim.y * 256) {
      float y = 0.f;
      for (int k = 0; k < K; ++k) y = y + O[(size_t)srow[k] * D + c] * sw[k];
      Y[c] = y + SH[c];
    }
  }
}

// One wave per (token, 128 columns): scale = amax / 448 (1 when amax = 0), codes = e4m3(x / scale).
__global__ __launch_bounds__(256) void act_quant(const bf16_t* __restrict__ x, uint8_t* __restrict__ xq,
                                                 float* __restrict__ sx, int64_t nblocks) {
#pragma clang fp contract(off)
  const int64_t gw = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (gw >= nblocks) return;
  const uint32_t p = *reinterpret_cast<const uint32_t*>(x + gw * 128 + lane * 2);
  const float a = bf16_to_f32((bf16_t)(p & 0xFFFF)), b = bf16_to_f32((bf16_t)(p >> 16));
  const float am = wave_max(fmaxf(fabsf(a), fabsf(b)));
  const float scale = am > 0.f ? am / 448.0f : 1.0f;
  const uint32_t q = f32x2_to_e4m3(a / scale, b / scale);
  *reinterpret_cast<uint16_t*>(xq + gw * 128 + lane * 2) = (uint16_t)q;
  if (lane == 0) sx[gw] = scale;
}

hipError_t launch_combine(const Dims& d, const int32_t* idx, const float* w, const int32_t* row_of,
                          const void* o_routed, const void* o_shared, void* out, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  // split the columns over more blocks when there are few tokens
  const unsigned ysplit = d.T >= 1024 ? 1u : (unsigned)std::max(1, std::min(8, d.D / 2048));
  if (d.dtype == 0)
    MOE_LAUNCH(combine<false>, dim3((unsigned)d.T, ysplit), dim3(256), 0, s, idx, w, row_of, o_routed, o_shared,
               out, d.K, d.D);
  else
    MOE_LAUNCH(combine<true>, dim3((unsigned)d.T, ysplit), dim3(256), 0, s, idx, w, row_of, o_routed, o_shared,
               out, d.K, d.D);
  return hipGetLastError();
}

hipError_t launch_act_quant(const Dims& d, const bf16_t* x, uint8_t* xq, float* sx, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  int64_t nb = d.T * (d.D / 128);
  MOE_LAUNCH(act_quant, dim3((unsigned)((nb + 3) / 4)), dim3(256), 0, s, x, xq, sx, nb);
  return hipGetLastError();
}

}  // namespace moe

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

// One block of CT threads per token (or per token and column slice when there are few tokens).
// The token's (expert, weight, row) triples are put in expert order by rank (experts of a token
// are distinct); each thread then owns 8-column chunks: it loads every routed row of its chunk
// (nontemporal: each row is read once) and the shared row before the in-order accumulation.
constexpr int CT = 128;

template <bool kBf16>
__global__ __launch_bounds__(CT) void combine(const int32_t* __restrict__ idx, const float* __restrict__ w,
                                              const int32_t* __restrict__ row_of, const void* __restrict__ o_routed,
                                              const void* __restrict__ o_shared, void* __restrict__ out, int K,
                                              int D) {
#pragma clang fp contract(off)
  __shared__ int srow[kMaxTopK];
  __shared__ float sw[kMaxTopK];
  const int t = blockIdx.x;
  if (threadIdx.x < K) {
    const int k = threadIdx.x;
    const int e = idx[(size_t)t * K + k];
    int rank = 0;
    for (int j = 0; j < K; ++j) {
      const int ej = idx[(size_t)t * K + j];
      rank += ej < e || (ej == e && j < k);
    }
    srow[rank] = row_of[(size_t)t * K + k];
    sw[rank] = w[(size_t)t * K + k];
  }
  __syncthreads();
  if (kBf16) {
    const bf16_t* O = static_cast<const bf16_t*>(o_routed);
    const bf16_t* SH = static_cast<const bf16_t*>(o_shared) + (size_t)t * D;
    bf16_t* Y = static_cast<bf16_t*>(out) + (size_t)t * D;
    for (int c = (blockIdx.y * CT + threadIdx.x) * 8; c < D; c += gridDim.y * CT * 8) {
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = 0.f;
      // all rows are loaded before the in-order accumulation
      i32x4 rows[kMaxTopK];
#pragma unroll
      for (int k = 0; k < kMaxTopK; ++k) {
        rows[k] = i32x4{0, 0, 0, 0};  // an assignment without a row (row_of < 0) adds zero
        if (k < K && srow[k] >= 0)
          rows[k] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(O + (size_t)srow[k] * D + c));
      }
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
    for (int c = blockIdx.y * CT + threadIdx.x; c < D; c += gridDim.y * CT) {
      float y = 0.f;
      for (int k = 0; k < K; ++k)
        if (srow[k] >= 0) y = y + O[(size_t)srow[k] * D + c] * sw[k];
      Y[c] = y + SH[c];
    }
  }
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

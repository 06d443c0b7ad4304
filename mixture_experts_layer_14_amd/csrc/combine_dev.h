// Device code of the combine shared by its kernel and the fused decode kernel ("DeepSeek-V3.2-Exp ·
// Mixture of experts", MoE.forward excerpt: an fp32 accumulator per token, the routed rows times
// their weights added in ascending expert order, then the shared expert's row).
#pragma once
#include "kernels.h"

namespace moe {

constexpr int kMaxTopK = 16;

// One block of CT threads per token (or per token and column slice when there are few tokens).
// The token's (expert, weight, row) triples are put in expert order by rank (experts of a token
// are distinct); each thread then owns 8-column chunks: it loads every routed row of its chunk
// (nontemporal: each row is read once) and the shared row before the in-order accumulation.
constexpr int CT = 128;

// Token t's columns yb * NT * 8 + ... on a block of NT threads (column slice yb of ny); srow and sw:
// kMaxTopK entries of LDS each.
template <bool kBf16, int NT>
MOE_DEV void combine_token(int t, int yb, int ny, int* srow, float* sw, const int32_t* __restrict__ idx,
                           const float* __restrict__ w, const int32_t* __restrict__ row_of,
                           const void* __restrict__ o_routed, const void* __restrict__ o_shared, void* __restrict__ out,
                           int K, int D) {
#pragma clang fp contract(off)
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
    for (int c = (yb * NT + threadIdx.x) * 8; c < D; c += ny * NT * 8) {
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
    for (int c = yb * NT + threadIdx.x; c < D; c += ny * NT) {
      float y = 0.f;
      for (int k = 0; k < K; ++k)
        if (srow[k] >= 0) y = y + O[(size_t)srow[k] * D + c] * sw[k];
      Y[c] = y + SH[c];
    }
  }
}

}  // namespace moe

// Router of the MoE block ("DeepSeek-V3.2-Exp · Router", formula steps 1-4 and the
// Gate.forward excerpt): logits, sigmoid, selection bias, group-limited top-k,
// renormalised and scaled weights.
#include <float.h>
#include <math.h>

#include <algorithm>

#include "router_dev.h"

namespace moe {

// Block: 4 waves on one tile of 32 tokens x 32 experts (logits_tile). Grid (T/32, E/32, nsplit).
__global__ __launch_bounds__(256) void router_logits_bf16(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wg,
                                                          double* __restrict__ zpart, int T, int D, int E,
                                                          int kslice) {
  __shared__ double red[3][16][64];
  logits_tile(x, wg, zpart, T, D, E, kslice, blockIdx.x, blockIdx.y, blockIdx.z, red);
}

// Large batches: a block holds 64 tokens x 256 experts over one k-slice, so x is read once per
// slice and W_r once per 64 tokens; wave w (of 8) takes tokens 32 (w / 4) .. + 31 and experts
// 64 (w % 4) .. + 63, chunks added in k order. Grid (T/64, E/256, nsplit).
__global__ __launch_bounds__(512) void router_logits_bf16_wide(const bf16_t* __restrict__ x,
                                                               const bf16_t* __restrict__ wg,
                                                               double* __restrict__ zpart, int T, int D, int E,
                                                               int kslice) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int split = blockIdx.z;
  const int kb = split * kslice, ke = min(D, kb + kslice);
  const int r = lane & 15, kq = lane >> 4;
  const int t0 = blockIdx.x * 64 + (wave >> 2) * 32;
  const int e0 = blockIdx.y * 256 + (wave & 3) * 64;
  const bf16_t* ap[2];
  bool av[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int t = t0 + m * 16 + r;
    av[m] = t < T;
    ap[m] = x + (size_t)(av[m] ? t : 0) * D + kq * 8;
  }
  const bf16_t* bp[4];
  bool bv[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int e = e0 + n * 16 + r;
    bv[n] = e < E;
    bp[n] = wg + (size_t)(bv[n] ? e : 0) * D + kq * 8;
  }
  double acc[2][4][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][n][i] = 0.0;
  const i32x4 zero = {0, 0, 0, 0};
  const f32x4 fz = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 4;  // chunks whose loads are issued together
  for (int k = kb; k < ke; k += 32 * U) {
    i32x4 a[U][2], b[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = k + 32 * u < ke;
#pragma unroll
      for (int m = 0; m < 2; ++m) a[u][m] = (av[m] && in) ? ld16(ap[m] + k + 32 * u) : zero;
#pragma unroll
      for (int n = 0; n < 4; ++n) b[u][n] = (bv[n] && in) ? ld16(bp[n] + k + 32 * u) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const f32x4 p = mfma_bf16_16x16x32(a[u][m], b[u][n], fz);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][n][i] += (double)p[i];
        }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int e = e0 + n * 16 + r;
      if (e >= E) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + m * 16 + kq * 4 + i;
        if (t < T) zpart[((size_t)split * T + t) * E + e] = acc[m][n][i];
      }
    }
}

// fp32 inputs: each product is exact in fp64; one thread per (token, expert).
__global__ __launch_bounds__(256) void router_logits_f32(const float* __restrict__ x, const float* __restrict__ wg,
                                                         double* __restrict__ zpart, int T, int D, int E) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * E) return;
  int t = (int)(i / E), e = (int)(i % E);
  const float* xr = x + (size_t)t * D;
  const float* wr = wg + (size_t)e * D;
  double acc = 0.0;
  for (int k = 0; k < D; ++k) acc += (double)xr[k] * (double)wr[k];
  zpart[i] = acc;
}

template <int EPT, int TPB>
__global__ __launch_bounds__(256) void router_select(const double* __restrict__ zpart, int nsplit,
                                                     const float* __restrict__ bias, int T, int E, int G, int Gk,
                                                     int K, float route_scale, int softmax,
                                                     int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  __shared__ SelectLds<EPT, TPB, 256 / TPB> L;
  select_block<EPT, TPB, 256>(blockIdx.x, zpart, nsplit, bias, T, E, G, Gk, K, route_scale, softmax, idx_out, w_out, L);
}

// Batches of 1024 tokens or more use the 64 x 256 tiles.
static bool router_wide(const Dims& d) { return d.dtype != 0 && d.T >= 1024; }

int router_splits(const Dims& d) {
  if (d.dtype == 0 || d.T == 0) return 1;
  const bool wide = router_wide(d);
  int64_t tiles = wide ? ((d.T + 63) / 64) * ((d.E + 255) / 256) : ((d.T + 31) / 32) * ((d.E + 31) / 32);
  // enough blocks to stream the router weight with many CUs, but few slices to add up, each
  // at least one chunk per wave
  int64_t want = (256 + tiles - 1) / tiles;
  int64_t max_split = std::min<int64_t>(kMaxSplit, d.D / (wide ? 64 : 128));
  if (want > max_split) want = max_split;
  if (want < 1) want = 1;
  return (int)want;
}

int router_kslice(const Dims& d, int nsplit) {
  int chunks = d.D / 32;
  return ((chunks + nsplit - 1) / nsplit) * 32;
}

hipError_t launch_router_logits(const Dims& d, const void* x, const void* w_gate, double* zpart, int nsplit,
                                hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  if (d.dtype == 0) {
    int64_t n = d.T * d.E;
    MOE_LAUNCH(router_logits_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float*)x, (const float*)w_gate, zpart, (int)d.T, d.D, d.E);
  } else {
    const int kslice = router_kslice(d, nsplit);
    if (router_wide(d)) {
      dim3 grid((unsigned)((d.T + 63) / 64), (unsigned)((d.E + 255) / 256), (unsigned)nsplit);
      MOE_LAUNCH(router_logits_bf16_wide, grid, dim3(512), 0, s, (const bf16_t*)x, (const bf16_t*)w_gate, zpart,
                 (int)d.T, d.D, d.E, kslice);
    } else {
      dim3 grid((unsigned)((d.T + 31) / 32), (unsigned)((d.E + 31) / 32), (unsigned)nsplit);
      MOE_LAUNCH(router_logits_bf16, grid, dim3(256), 0, s, (const bf16_t*)x, (const bf16_t*)w_gate, zpart,
                 (int)d.T, d.D, d.E, kslice);
    }
  }
  return hipGetLastError();
}

hipError_t launch_router_select(const Dims& d, const double* zpart, int nsplit, const float* bias,
                                float route_scale, bool softmax, int32_t* idx, float* w, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  // the selection kernel's per-token arrays are sized for these limits (the ABI rejects larger
  // configurations before any launch)
  if (d.E > kMaxE || d.G > kMaxG || d.K > kMaxK || nsplit > kMaxSplit) return hipErrorInvalidValue;
  // one token per block for small batches (latency), one per wave for large ones with E <= 256
#define MOE_SELECT(EPT, TPB)                                                                              \
  MOE_LAUNCH((router_select<EPT, TPB>), dim3((unsigned)((d.T + TPB - 1) / TPB)), dim3(256), 0, s, zpart, nsplit, \
             bias, (int)d.T, d.E, d.G, d.Gk, d.K, route_scale, softmax ? 1 : 0, idx, w)
  if (d.T > 256 && d.E <= 64) MOE_SELECT(1, 4);
  else if (d.T > 256 && d.E <= 128) MOE_SELECT(2, 4);
  else if (d.T > 256 && d.E <= 256) MOE_SELECT(4, 4);
  else if (d.E <= 256) MOE_SELECT(1, 1);
  else if (d.E <= 512) MOE_SELECT(2, 1);
  else MOE_SELECT(4, 1);
#undef MOE_SELECT
  return hipGetLastError();
}

}  // namespace moe

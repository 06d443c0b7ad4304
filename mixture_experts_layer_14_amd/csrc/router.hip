// Router of the MoE block ("DeepSeek-V3.2-Exp · Router", formula steps 1-4 and the
// Gate.forward excerpt): logits, sigmoid, selection bias, group-limited top-k,
// renormalised and scaled weights.
#include <float.h>
#include <math.h>

#include <algorithm>

#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Step 1: z = x W_r^T. Each 32-wide k chunk is one bf16 MFMA (products exact in
// fp32, chunk sum rounded once) and the chunks are summed in fp64, so z keeps
// well under 1e-7 absolute error before its single rounding to fp32. Partial
// sums over `nsplit` slices of D are written to zpart[split][T][E] (fp64) and
// added in split order by router_reduce.
//
// Block: 4 waves; wave tile 32 tokens x 32 experts (2 x 2 MFMA tiles); block
// tile 32 tokens x 128 experts. Grid (T/32, E/128, nsplit).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_logits_bf16(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wg,
                                                          double* __restrict__ zpart, int T, int D, int E,
                                                          int kslice) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, kq = lane >> 4;
  const int t0 = blockIdx.x * 32;
  const int e0 = blockIdx.y * 128 + wave * 32;
  const int split = blockIdx.z;
  const int kb = split * kslice;
  const int ke = min(D, kb + kslice);

  const bf16_t* ap[2];
  bool av[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    int t = t0 + m * 16 + r;
    av[m] = t < T;
    ap[m] = x + (size_t)(av[m] ? t : 0) * D + kq * 8;
  }
  const bf16_t* bp[2];
  bool bv[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    int e = e0 + n * 16 + r;
    bv[n] = e < E;
    bp[n] = wg + (size_t)(bv[n] ? e : 0) * D + kq * 8;
  }
  double acc[2][2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][n][i] = 0.0;

  const i32x4 zero = {0, 0, 0, 0};
  const f32x4 fz = {0.f, 0.f, 0.f, 0.f};
  for (int k = kb; k < ke; k += 32) {
    i32x4 a[2], b[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) a[m] = av[m] ? ld16(ap[m] + k) : zero;
#pragma unroll
    for (int n = 0; n < 2; ++n) b[n] = bv[n] ? ld16(bp[n] + k) : zero;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f32x4 p = mfma_bf16_16x16x32(a[m], b[n], fz);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][n][i] += (double)p[i];
      }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      int e = e0 + n * 16 + r;
      if (e >= E) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int t = t0 + m * 16 + kq * 4 + i;
        if (t < T) zpart[((size_t)split * T + t) * E + e] = acc[m][n][i];
      }
    }
}

// Sum the per-slice fp64 partial logits in slice order and round once to fp32.
__global__ __launch_bounds__(256) void router_reduce(const double* __restrict__ zpart, int nsplit, int64_t n,
                                                     float* __restrict__ z) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  double part[16];
#pragma unroll
  for (int p = 0; p < 16; ++p) part[p] = p < nsplit ? zpart[(size_t)p * n + i] : 0.0;
  double acc = 0.0;
#pragma unroll
  for (int p = 0; p < 16; ++p)
    if (p < nsplit) acc += part[p];
  z[i] = (float)acc;
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

// ---------------------------------------------------------------------------
// Steps 2-4, one wave per token. Per-wave LDS: s[E], sb[E], group scores, keep flags.
// Ties everywhere resolve to the lower index; the chosen experts come out in
// descending selection score.
// ---------------------------------------------------------------------------
constexpr int kMaxE = 1024, kMaxG = 64, kMaxK = 16;

__global__ __launch_bounds__(256) void router_select(const double* __restrict__ zpart, const float* __restrict__ z32,
                                                     const float* __restrict__ bias, int T, int E, int G, int Gk,
                                                     int K, float route_scale, int32_t* __restrict__ idx_out,
                                                     float* __restrict__ w_out) {
#pragma clang fp contract(off)
  extern __shared__ float smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  const bool active = t < T;
  float* s = smem + wave * (2 * E + 2 * kMaxG);
  float* sb = s + E;
  float* gsc = sb + E;
  int* keep = reinterpret_cast<int*>(gsc + kMaxG);
  const int gsize = E / G;

  if (active) {
    for (int e = lane; e < E; e += 64) {
      const float zf = z32 ? z32[(size_t)t * E + e] : (float)zpart[(size_t)t * E + e];
      float sv = (float)(1.0 / (1.0 + exp(-(double)zf)));
      s[e] = sv;
      sb[e] = bias ? sv + bias[e] : sv;
    }
  }
  __syncthreads();
  if (active && lane < G) {
    float best = -INFINITY, second = -INFINITY;
    const float* v = sb + lane * gsize;
    for (int i = 0; i < gsize; ++i) {
      float q = v[i];
      if (q > best) {
        second = best;
        best = q;
      } else if (q > second) {
        second = q;
      }
    }
    gsc[lane] = bias ? best + second : best;
  }
  __syncthreads();
  if (active && lane < G) {
    float mine = gsc[lane];
    int rank = 0;
    for (int g = 0; g < G; ++g) {
      float o = gsc[g];
      rank += (o > mine) || (o == mine && g < lane);
    }
    keep[lane] = (G == 1) || rank < Gk;
  }
  __syncthreads();
  if (!active) return;

  // masked selection scores owned by this lane: experts lane, lane + 64, ...
  float m[kMaxE / 64];
  uint32_t taken = 0;
  const int nper = (E + 63) / 64;
#pragma unroll
  for (int j = 0; j < kMaxE / 64; ++j) {
    int e = lane + 64 * j;
    m[j] = (j < nper && e < E && keep[e / gsize]) ? sb[e] : -INFINITY;
  }
  int sel[kMaxK];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    if (k >= K) continue;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kMaxE / 64; ++j) {
      int e = lane + 64 * j;
      if (j < nper && e < E && !((taken >> j) & 1u) && (m[j] > bv || (m[j] == bv && e < bi))) {
        bv = m[j];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(bv, off);
      int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    sel[k] = bi;
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
  }
  // weights: unbiased scores of the chosen experts, divided by their rank-order sum, scaled
  float tot = s[sel[0]];
#pragma unroll
  for (int k = 1; k < kMaxK; ++k)
    if (k < K) tot = tot + s[sel[k]];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    if (k < K && lane == k) {
      float wk = s[sel[k]] / tot;
      idx_out[(size_t)t * K + k] = sel[k];
      w_out[(size_t)t * K + k] = wk * route_scale;
    }
  }
}

int router_splits(const Dims& d) {
  if (d.dtype == 0) return 1;
  int64_t row_tiles = (d.T + 31) / 32;
  int64_t col_tiles = (d.E + 127) / 128;
  // enough blocks to stream the router weight with many CUs, but few slices to add up
  int64_t want = (256 + row_tiles * col_tiles - 1) / (row_tiles * col_tiles);
  int64_t max_split = std::min<int64_t>(16, d.D / 64);
  if (want > max_split) want = max_split;
  if (want < 1) want = 1;
  return (int)want;
}

static int split_len(const Dims& d, int nsplit) {
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
    int kslice = split_len(d, nsplit);
    dim3 grid((unsigned)((d.T + 31) / 32), (unsigned)((d.E + 127) / 128), (unsigned)nsplit);
    MOE_LAUNCH(router_logits_bf16, grid, dim3(256), 0, s, (const bf16_t*)x, (const bf16_t*)w_gate,
                       zpart, (int)d.T, d.D, d.E, kslice);
  }
  return hipGetLastError();
}

hipError_t launch_router_select(const Dims& d, const double* zpart, int nsplit, float* z32, const float* bias,
                                float route_scale, int32_t* idx, float* w, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  const float* zf = nullptr;
  if (nsplit > 1) {
    int64_t n = d.T * d.E;
    MOE_LAUNCH(router_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, zpart, nsplit, n, z32);
    zf = z32;
  }
  size_t lds = 4 * (2 * (size_t)d.E + 2 * kMaxG) * sizeof(float);
  MOE_LAUNCH(router_select, dim3((unsigned)((d.T + 3) / 4)), dim3(256), lds, s, zpart, zf, bias,
                     (int)d.T, d.E, d.G, d.Gk, d.K, route_scale, idx, w);
  return hipGetLastError();
}

}  // namespace moe

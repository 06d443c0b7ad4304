// Routed and shared SwiGLU experts ("DeepSeek-V3.2-Exp · Mixture of experts": each expert
// is three dim x inter matrices; the parameter table counts 3 * 7168 * 2048 per expert):
//   h = silu(A W1^T) * (A W3^T)      (gate/up GEMM with the SwiGLU epilogue)
//   O = h W2^T                       (down GEMM)
// A is x gathered through the dispatch permutation (routed rows) or x itself (shared
// expert, tile expert index E). Work comes from the device-side tile lists the dispatch
// wrote, so experts with no tokens are never read and the host never waits.
#include <algorithm>

#include "kernels.h"

namespace moe {

constexpr int kPersistBlocks = 256 * 8;  // grid cap of the fp32 kernels

__device__ __forceinline__ int n_items(const int32_t* meta, int list, int per_routed, int per_shared) {
  int nr = meta[2 * list], na = meta[2 * list + 1];
  return nr * per_routed + (na - nr) * per_shared;
}

// item -> (tile index, n-tile index)
__device__ __forceinline__ void split_item(int item, const int32_t* meta, int list, int per_routed, int per_shared,
                                           int* tile, int* nt) {
  int nr = meta[2 * list];
  int routed_items = nr * per_routed;
  if (item < routed_items) {
    *tile = item / per_routed;
    *nt = item % per_routed;
  } else {
    int j = item - routed_items;
    *tile = nr + j / per_shared;
    *nt = j % per_shared;
  }
}

// ===========================================================================
// fp8 (e4m3fn, 128x128 weight blocks, 1x128 activation blocks), M-tiles of 16 rows.
// One K=128 MFMA covers exactly one scale block; its partial sum is scaled by
// sx(row) * sw(block) in fp32 and accumulated.
// ===========================================================================

// Item: 16 rows x 128 h-columns (one activation scale block), 4 waves x 32 columns, full K.
// Epilogue: h = silu(g) * u, then per row amax over the 128 columns, scale = amax / 448,
// codes = e4m3(h / scale).
__global__ __launch_bounds__(256) void gemm1_fp8_m16(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
                                                     const int32_t* __restrict__ row_token,
                                                     const Tile* __restrict__ tiles, const int32_t* __restrict__ meta,
                                                     const uint8_t* __restrict__ w1, const uint8_t* __restrict__ w3,
                                                     const float* __restrict__ s1, const float* __restrict__ s3,
                                                     const uint8_t* __restrict__ ws1, const uint8_t* __restrict__ ws3,
                                                     const float* __restrict__ ss1, const float* __restrict__ ss3,
                                                     uint8_t* __restrict__ h_routed, float* __restrict__ h_scale,
                                                     uint8_t* __restrict__ h_shared, float* __restrict__ h_shared_scale,
                                                     int D, int I, int S, int E) {
#pragma clang fp contract(off)
  __shared__ float hbuf[16][129];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, kq = lane >> 4;
  const int per_r = I / 128, per_s = S / 128;
  const int items = n_items(meta, 0, per_r, per_s);
  const int KB = D / 128;
  const i32x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
  const f32x4 fz = {0.f, 0.f, 0.f, 0.f};
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    int ti, nt;
    split_item(item, meta, 0, per_r, per_s, &ti, &nt);
    const Tile tl = tiles[ti];
    const bool sh = tl.expert == E;
    const int NI = sh ? S : I;
    const uint8_t* W1 = sh ? ws1 : w1 + (size_t)tl.expert * I * D;
    const uint8_t* W3 = sh ? ws3 : w3 + (size_t)tl.expert * I * D;
    const float* S1 = (sh ? ss1 : s1 + (size_t)tl.expert * (I / 128) * KB) + (size_t)nt * KB;
    const float* S3 = (sh ? ss3 : s3 + (size_t)tl.expert * (I / 128) * KB) + (size_t)nt * KB;
    const int n0 = nt * 128 + wave * 32;
    // A operand row of this lane, and the x scales of the 4 accumulator rows of this lane
    const bool av = r < tl.nrows;
    int tok = 0;
    if (av) tok = sh ? tl.row0 + r : row_token[tl.row0 + r];
    const float* sxr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int row = kq * 4 + i;
      int tk = 0;
      if (row < tl.nrows) tk = sh ? tl.row0 + row : row_token[tl.row0 + row];
      sxr[i] = sx + (size_t)tk * KB;
    }
    const uint8_t* ap = xq + (size_t)tok * D + kq * 32;
    const uint8_t* bp1[2];
    const uint8_t* bp3[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bp1[j] = W1 + (size_t)(n0 + j * 16 + r) * D + kq * 32;
      bp3[j] = W3 + (size_t)(n0 + j * 16 + r) * D + kq * 32;
    }
    f32x4 g[2] = {fz, fz}, u[2] = {fz, fz};
    for (int kb = 0; kb < KB; ++kb) {
      const int k = kb * 128;
      i32x8 a = av ? ld32(ap + k) : zero;
      i32x8 b1[2], b3[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        b1[j] = ld32(bp1[j] + k);
        b3[j] = ld32(bp3[j] + k);
      }
      const float sw1 = S1[kb], sw3 = S3[kb];
      float sxv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sxv[i] = sxr[i][kb];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f32x4 p1 = mfma_fp8_16x16x128(a, b1[j], fz);
        f32x4 p3 = mfma_fp8_16x16x128(a, b3[j], fz);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          g[j][i] += p1[i] * (sxv[i] * sw1);
          u[j][i] += p3[i] * (sxv[i] * sw3);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) hbuf[kq * 4 + i][wave * 32 + j * 16 + r] = silu_mul(g[j][i], u[j][i]);
    __syncthreads();
    {
      // 16 threads per row, 8 columns each
      const int row = threadIdx.x >> 4, c = (threadIdx.x & 15) * 8;
      float v[8];
      float am = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        v[q] = hbuf[row][c + q];
        am = fmaxf(am, fabsf(v[q]));
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
      const float scale = am > 0.f ? am / 448.0f : 1.0f;
      if (row < tl.nrows) {
        uint32_t lo = f32x2_to_e4m3(v[0] / scale, v[1] / scale) | (f32x2_to_e4m3(v[2] / scale, v[3] / scale) << 16);
        uint32_t hi = f32x2_to_e4m3(v[4] / scale, v[5] / scale) | (f32x2_to_e4m3(v[6] / scale, v[7] / scale) << 16);
        uint8_t* dst = sh ? h_shared + (size_t)(tl.row0 + row) * S : h_routed + (size_t)(tl.row0 + row) * I;
        *reinterpret_cast<uint2*>(dst + nt * 128 + c) = make_uint2(lo, hi);
        if ((threadIdx.x & 15) == 0) {
          float* sd = sh ? h_shared_scale + (size_t)(tl.row0 + row) * (S / 128)
                         : h_scale + (size_t)(tl.row0 + row) * (I / 128);
          sd[nt] = scale;
        }
      }
    }
    (void)NI;
    __syncthreads();
  }
}

// Item: 16 rows x 64 output columns (4 waves x 16), full K = I in 128-blocks.
__global__ __launch_bounds__(256) void gemm2_fp8_m16(const uint8_t* __restrict__ h_routed,
                                                     const float* __restrict__ h_scale,
                                                     const uint8_t* __restrict__ h_shared,
                                                     const float* __restrict__ h_shared_scale,
                                                     const Tile* __restrict__ tiles, const int32_t* __restrict__ meta,
                                                     const uint8_t* __restrict__ w2, const float* __restrict__ s2,
                                                     const uint8_t* __restrict__ ws2, const float* __restrict__ ss2,
                                                     bf16_t* __restrict__ o_routed, bf16_t* __restrict__ o_shared,
                                                     int D, int I, int S, int E) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, kq = lane >> 4;
  const int per = D / 64;
  const int items = n_items(meta, 0, per, per);
  const i32x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
  const f32x4 fz = {0.f, 0.f, 0.f, 0.f};
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    int ti, nt;
    split_item(item, meta, 0, per, per, &ti, &nt);
    const Tile tl = tiles[ti];
    const bool sh = tl.expert == E;
    const int KK = sh ? S : I;
    const int KB = KK / 128;
    const uint8_t* A = sh ? h_shared + (size_t)tl.row0 * S : h_routed + (size_t)tl.row0 * I;
    const float* AS = sh ? h_shared_scale + (size_t)tl.row0 * KB : h_scale + (size_t)tl.row0 * KB;
    const uint8_t* W = sh ? ws2 : w2 + (size_t)tl.expert * D * I;
    const int c0 = nt * 64 + wave * 16;
    const float* SW = (sh ? ss2 : s2 + (size_t)tl.expert * (D / 128) * KB) + (size_t)(c0 / 128) * KB;
    const bool av = r < tl.nrows;
    const uint8_t* ap = A + (size_t)(av ? r : 0) * KK + kq * 32;
    const uint8_t* bp = W + (size_t)(c0 + r) * KK + kq * 32;
    int srow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) srow[i] = min(kq * 4 + i, tl.nrows - 1);
    f32x4 acc = fz;
    for (int kb = 0; kb < KB; ++kb) {
      const int k = kb * 128;
      i32x8 a = av ? ld32(ap + k) : zero;
      i32x8 b = ld32(bp + k);
      f32x4 p = mfma_fp8_16x16x128(a, b, fz);
      const float sw = SW[kb];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += p[i] * (AS[(size_t)srow[i] * KB + kb] * sw);
    }
    bf16_t* O = sh ? o_shared : o_routed;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int row = kq * 4 + i;
      if (row < tl.nrows) O[(size_t)(tl.row0 + row) * D + c0 + r] = f32_to_bf16(acc[i]);
    }
  }
}

// ===========================================================================
// fp32 (small blocks): one thread per output element, fp32 fused multiply-adds.
// ===========================================================================
__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int row) {
  int lo = 0, hi = E;  // largest e with offsets[e] <= row
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (offsets[mid] <= row) lo = mid;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void gemm1_f32(const float* __restrict__ x, const int32_t* __restrict__ row_token,
                                                 const int32_t* __restrict__ offsets, const float* __restrict__ w1,
                                                 const float* __restrict__ w3, const float* __restrict__ ws1,
                                                 const float* __restrict__ ws3, float* __restrict__ h_routed,
                                                 float* __restrict__ h_shared, int64_t R, int64_t T, int D, int I, int S,
                                                 int E) {
  const int64_t total = R * I + T * S;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const float *xr, *a1, *a3;
    float* dst;
    if (i < R * I) {
      int row = (int)(i / I), n = (int)(i % I);
      int e = expert_of_row(offsets, E, row);
      xr = x + (size_t)row_token[row] * D;
      a1 = w1 + ((size_t)e * I + n) * D;
      a3 = w3 + ((size_t)e * I + n) * D;
      dst = h_routed + i;
    } else {
      int64_t j = i - R * I;
      int tok = (int)(j / S), n = (int)(j % S);
      xr = x + (size_t)tok * D;
      a1 = ws1 + (size_t)n * D;
      a3 = ws3 + (size_t)n * D;
      dst = h_shared + j;
    }
    float g = 0.f, u = 0.f;
    for (int k = 0; k < D; ++k) {
      g = fmaf(xr[k], a1[k], g);
      u = fmaf(xr[k], a3[k], u);
    }
    *dst = silu_mul(g, u);
  }
}

__global__ __launch_bounds__(256) void gemm2_f32(const float* __restrict__ h_routed, const float* __restrict__ h_shared,
                                                 const int32_t* __restrict__ offsets, const float* __restrict__ w2,
                                                 const float* __restrict__ ws2, float* __restrict__ o_routed,
                                                 float* __restrict__ o_shared, int64_t R, int64_t T, int D, int I, int S,
                                                 int E) {
  const int64_t total = (R + T) * D;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    int64_t row = i / D;
    int c = (int)(i % D);
    const float *hr, *wr;
    int KK;
    float* dst;
    if (row < R) {
      int e = expert_of_row(offsets, E, (int)row);
      hr = h_routed + (size_t)row * I;
      wr = w2 + ((size_t)e * D + c) * I;
      KK = I;
      dst = o_routed + i;
    } else {
      hr = h_shared + (size_t)(row - R) * S;
      wr = ws2 + (size_t)c * S;
      KK = S;
      dst = o_shared + (i - R * D);
    }
    float acc = 0.f;
    for (int k = 0; k < KK; ++k) acc = fmaf(hr[k], wr[k], acc);
    *dst = acc;
  }
}

static unsigned grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  return (unsigned)(b < kPersistBlocks ? (b < 1 ? 1 : b) : kPersistBlocks);
}

hipError_t launch_experts(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  const int E = d.E;
  if (d.dtype == 0) {
    MOE_LAUNCH(gemm1_f32, dim3(grid_for(d.R * d.I + d.T * d.S)), dim3(256), 0, s, (const float*)a.x,
                       a.row_token, a.offsets, (const float*)w.w1, (const float*)w.w3, (const float*)w.ws1,
                       (const float*)w.ws3, (float*)a.h_routed, (float*)a.h_shared, d.R, d.T, d.D, d.I, d.S, E);
    MOE_LAUNCH(gemm2_f32, dim3(grid_for((d.R + d.T) * d.D)), dim3(256), 0, s, (const float*)a.h_routed,
                       (const float*)a.h_shared, a.offsets, (const float*)w.w2, (const float*)w.ws2,
                       (float*)a.o_routed, (float*)a.o_shared, d.R, d.T, d.D, d.I, d.S, E);
    return hipGetLastError();
  }
  // 128-row tiles once the routed experts average 16 rows or more; for a dense feed-forward (no
  // routed experts) once it has kDenseWideRows tokens
  const bool wide = d.E > 0 ? d.R >= 16 * (int64_t)d.E : d.T >= kDenseWideRows;
  if (d.dtype == 1) {
    if (wide_ok(d) && wide) return launch_wide_bf16(d, w, a, s);
    return launch_stream_bf16(d, w, a, s);
  }
  if (wide) {
    if (wstream_fp8_ok(d)) return launch_wstream_fp8(d, w, a, s);
    if (wide_fp8_ok(d)) return launch_wide_fp8(d, w, a, s);
  }
  const int g1 = persistent_grid((const void*)gemm1_fp8_m16, 256);
  const int g2 = persistent_grid((const void*)gemm2_fp8_m16, 256);
  MOE_LAUNCH(gemm1_fp8_m16, dim3(g1), dim3(256), 0, s,
                     (const uint8_t*)a.x, a.x_scale, a.row_token, a.tiles_skinny, a.meta, (const uint8_t*)w.w1,
                     (const uint8_t*)w.w3, w.s1, w.s3, (const uint8_t*)w.ws1, (const uint8_t*)w.ws3, w.ss1, w.ss3,
                     (uint8_t*)a.h_routed, a.h_scale, (uint8_t*)a.h_shared, a.h_shared_scale, d.D, d.I, d.S, E);
  MOE_LAUNCH(gemm2_fp8_m16, dim3(g2), dim3(256), 0, s,
                     (const uint8_t*)a.h_routed, a.h_scale, (const uint8_t*)a.h_shared, a.h_shared_scale,
                     a.tiles_skinny, a.meta, (const uint8_t*)w.w2, w.s2, (const uint8_t*)w.ws2, w.ss2,
                     (bf16_t*)a.o_routed, (bf16_t*)a.o_shared, d.D, d.I, d.S, E);
  return hipGetLastError();
}

}  // namespace moe

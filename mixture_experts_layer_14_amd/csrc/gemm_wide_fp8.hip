// Prefill-sized expert GEMMs in FP8 (OCP e4m3fn) with fine-grained scales: weights carry one
// fp32 scale per 128x128 block of the [out, in] matrix, activations one per row per 128
// columns. The SwiGLU expert of "DeepSeek-V3.2-Exp · Mixture of experts":
//   mode 0 (gate/up): h = silu(A W1^T) * (A W3^T), then h is quantised per row per 128
//                     columns (scale = amax / 448, 1 if amax = 0) in the epilogue
//   mode 1 (down):    O = h W2^T in bf16
//
// A k-stage is exactly one scale block (128 k). Its partial products come from two
// 32x32x64 fp8 MFMAs started from zero and are added to the fp32 accumulators times
// sx(row, kb) * sw(n-block, kb). Tiles: 128 rows x (mode 0: 128 h-columns = 128 rows of W1
// and the same 128 rows of W3; mode 1: 128 output columns), so every tile column lies in a
// single weight scale block and, in mode 0, every h row segment of the tile is one
// activation scale block. Mode 0 runs 8 waves (2 row halves x 4 column quarters, each with
// the gate and up accumulators of the same 32 h-columns); mode 1 runs 4 waves (2 x 2).
// Operand tiles are staged through XOR-swizzled LDS (128-byte rows) while the next stage is
// in flight in registers; the 128 row scales of each stage go to LDS with it. Items and the XCD-aware persistent grid are as in the bf16 wide kernels.
#include "kernels.h"

namespace moe {

constexpr int FBM = kWideBM;  // 128 rows
constexpr int FBK = 128;      // one scale block

// D(32x32, fp32) += A(32x64) * B(64x32), e4m3 with unit block scales (E8M0 127 = 1.0).
// Lane l holds A row / B column (l % 32) and 32 consecutive k of half (l / 32).
MOE_DEV f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

MOE_DEV i32x8 lds_frag32(const char* base, int row, int c0) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(base + swz(row, c0));
  const i32x4 hi = *reinterpret_cast<const i32x4*>(base + swz(row, c0 + 1));
  i32x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return r;
}

template <int MODE>
__global__ __launch_bounds__(MODE == 0 ? 512 : 256, 2) void gemm_wide_fp8(
    const uint8_t* __restrict__ aq, const float* __restrict__ a_scale,   // mode 0: xq [T, D], sx [T, D/128]
    const uint8_t* __restrict__ h_routed_in, const float* __restrict__ hs_routed_in,
    const uint8_t* __restrict__ h_shared_in, const float* __restrict__ hs_shared_in,
    const int32_t* __restrict__ row_token, const int32_t* __restrict__ offsets, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ meta, const uint8_t* __restrict__ wa, const uint8_t* __restrict__ wb,
    const float* __restrict__ sa, const float* __restrict__ sb, const uint8_t* __restrict__ wsa,
    const uint8_t* __restrict__ wsb, const float* __restrict__ ssa, const float* __restrict__ ssb,
    void* __restrict__ out_routed, float* __restrict__ outs_routed, void* __restrict__ out_shared,
    float* __restrict__ outs_shared, int T, int D, int I, int S, int E) {
  constexpr int THREADS = MODE == 0 ? 512 : 256;
  constexpr int NWN = MODE == 0 ? 4 : 2;       // waves across the tile columns
  constexpr int RPL = THREADS / 8;             // rows per load pass (8 threads per 128-byte row)
  constexpr int NAL = FBM / RPL;               // A loads per thread per stage
  constexpr int NB = MODE == 0 ? 256 : 128;    // weight rows per tile
  constexpr int NBL = NB / RPL;                // B loads per thread per stage
  __shared__ __attribute__((aligned(16))) char smem[(FBM + NB) * 128];
  __shared__ float sxs[FBM];
  __shared__ float amax_part[NWN][FBM];
  char* As = smem;
  char* Bs = smem + FBM * 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int l32 = lane & 31, lh = lane >> 5;
  const int ldr = tid >> 3, ldc = tid & 7;

  const int per_r = MODE == 0 ? I / 128 : D / 128;
  const int per_s = MODE == 0 ? S / 128 : D / 128;
  const int items = meta[2] * per_r + (meta[3] - meta[2]) * per_s;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
  const int chunk = (items + 7) >> 3;

  for (int j = slot; j < chunk; j += per_xcd) {
    const int item = xcd * chunk + j;
    if (item >= items) break;
    const WideItem it = wide_item(item, tiles, meta[2], offsets, T, E, per_r, per_s);
    const Tile tl = it.tl;
    const bool sh = it.shared;
    const int K = MODE == 0 ? D : (sh ? S : I);
    const int KB = K / FBK;

    // A rows of this thread's loads (clamped into the tile) and this thread's scale row
    const uint8_t* asrc[NAL];
#pragma unroll
    for (int i = 0; i < NAL; ++i) {
      const int r = min(ldr + RPL * i, tl.nrows - 1);
      if (MODE == 0) {
        const int tok = sh ? tl.row0 + r : row_token[tl.row0 + r];
        asrc[i] = aq + (size_t)tok * D + ldc * 16;
      } else {
        asrc[i] = (sh ? h_shared_in + (size_t)(tl.row0 + r) * S : h_routed_in + (size_t)(tl.row0 + r) * I) + ldc * 16;
      }
    }
    const float* srow = nullptr;  // thread t < 128 stages the scale of tile row t
    if (tid < FBM) {
      const int r = min(tid, tl.nrows - 1);
      if (MODE == 0) {
        const int tok = sh ? tl.row0 + r : row_token[tl.row0 + r];
        srow = a_scale + (size_t)tok * KB;
      } else {
        srow = sh ? hs_shared_in + (size_t)(tl.row0 + r) * KB : hs_routed_in + (size_t)(tl.row0 + r) * KB;
      }
    }
    // weight rows and the scale rows of the two matrices (mode 1: one)
    const uint8_t* Wa = sh ? wsa : wa + (size_t)tl.expert * (MODE == 0 ? (size_t)I * D : (size_t)D * I);
    const uint8_t* Wb = MODE == 0 ? (sh ? wsb : wb + (size_t)tl.expert * I * D) : nullptr;
    const int nblk_rows = (MODE == 0 ? (sh ? S : I) : D) / 128;  // 128-row scale blocks per matrix
    const float* Sa = (sh ? ssa : sa + (size_t)tl.expert * nblk_rows * KB) + (size_t)it.nt * KB;
    const float* Sb = MODE == 0 ? (sh ? ssb : sb + (size_t)tl.expert * nblk_rows * KB) + (size_t)it.nt * KB : nullptr;
    const uint8_t* bsrc[NBL];
#pragma unroll
    for (int i = 0; i < NBL; ++i) {
      const int br = ldr + RPL * i;
      if (MODE == 0) {
        const uint8_t* W = br < 128 ? Wa : Wb;
        bsrc[i] = W + (size_t)(it.nt * 128 + (br & 127)) * D + ldc * 16;
      } else {
        bsrc[i] = Wa + (size_t)(it.nt * 128 + br) * K + ldc * 16;
      }
    }

    constexpr int NT = 2;  // n sub-tiles of 32 per wave (mode 0: gate and up of the same 32 h-columns)
    f32x16 acc[2][NT];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < NT; ++b)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[a][b][q] = 0.f;

    i32x4 ra[NAL], rb[NBL];
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < NAL; ++i) ra[i] = ld16(asrc[i]);
#pragma unroll
    for (int i = 0; i < NBL; ++i) rb[i] = ld16(bsrc[i]);
    if (srow) rs = srow[0];
    const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    for (int kb = 0; kb < KB; ++kb) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NAL; ++i) *reinterpret_cast<i32x4*>(As + swz(ldr + RPL * i, ldc)) = ra[i];
#pragma unroll
      for (int i = 0; i < NBL; ++i) *reinterpret_cast<i32x4*>(Bs + swz(ldr + RPL * i, ldc)) = rb[i];
      if (tid < FBM) sxs[tid] = rs;
      __syncthreads();
      const float swa = Sa[kb];
      const float swb = MODE == 0 ? Sb[kb] : 0.f;
      if (kb + 1 < KB) {
        const int k = (kb + 1) * FBK;
#pragma unroll
        for (int i = 0; i < NAL; ++i) ra[i] = ld16(asrc[i] + k);
#pragma unroll
        for (int i = 0; i < NBL; ++i) rb[i] = ld16(bsrc[i] + k);
        if (srow) rs = srow[kb + 1];
      }
      i32x8 af[2][2], bfm[2][NT];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int c0 = kk * 4 + lh * 2;
#pragma unroll
        for (int m = 0; m < 2; ++m) af[kk][m] = lds_frag32(As, wm * 64 + m * 32 + l32, c0);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          // mode 0: n = 0 gate rows (W1 part), n = 1 the same h-columns of W3
          const int brow = MODE == 0 ? n * 128 + wn * 32 + l32 : wn * 64 + n * 32 + l32;
          bfm[kk][n] = lds_frag32(Bs, brow, c0);
        }
      }
      f32x16 p[2][NT];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n)
          p[m][n] = mfma32_fp8(af[1][m], bfm[1][n], mfma32_fp8(af[0][m], bfm[0][n], zero16));
      // scale promotion: rows of this lane are wm*64 + m*32 + 8 jj + 4 lh + i
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 sx4 = *reinterpret_cast<const f32x4*>(&sxs[wm * 64 + m * 32 + jj * 8 + lh * 4]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float fa = sx4[i] * swa;
            const int q = jj * 4 + i;
            if (MODE == 0) {
              const float fb = sx4[i] * swb;
              acc[m][0][q] += p[m][0][q] * fa;
              acc[m][1][q] += p[m][1][q] * fb;
            } else {
              acc[m][0][q] += p[m][0][q] * fa;
              acc[m][1][q] += p[m][1][q] * fa;
            }
          }
        }
      }
    }

    if (MODE == 1) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = wm * 64 + m * 32 + (q >> 2) * 8 + lh * 4 + (q & 3);
          if (row >= tl.nrows) continue;
          bf16_t* dst = static_cast<bf16_t*>(sh ? out_shared : out_routed) + (size_t)(tl.row0 + row) * D +
                        it.nt * 128 + wn * 64 + l32;
          dst[0] = f32_to_bf16(acc[m][0][q]);
          dst[32] = f32_to_bf16(acc[m][1][q]);
        }
      continue;
    }
    // mode 0 epilogue: h = silu(g) * u; per row amax over the tile's 128 h-columns; e4m3 codes.
    float hv[2][16];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int q = 0; q < 16; ++q) hv[m][q] = silu_mul(acc[m][0][q], acc[m][1][q]);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        float a = fabsf(hv[m][q]);
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));  // over the 32 columns
        const int row = wm * 64 + m * 32 + (q >> 2) * 8 + lh * 4 + (q & 3);
        if (l32 == 0) amax_part[wn][row] = a;
      }
    __syncthreads();  // amax parts visible; all waves are done reading the operand tiles
    char* Hs = smem;  // 128 rows x 128 code bytes, rows not swizzled
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = wm * 64 + m * 32 + (q >> 2) * 8 + lh * 4 + (q & 3);
        float am = amax_part[0][row];
#pragma unroll
        for (int w = 1; w < NWN; ++w) am = fmaxf(am, amax_part[w][row]);
        const float scale = am > 0.f ? am / 448.0f : 1.0f;
        Hs[row * 128 + wn * 32 + l32] = (char)(f32x2_to_e4m3(hv[m][q] / scale, 0.f) & 0xFF);
      }
    __syncthreads();
    uint8_t* Hout = static_cast<uint8_t*>(sh ? out_shared : out_routed);
    float* Sout = sh ? outs_shared : outs_routed;
    const int ldh = sh ? S : I;
#pragma unroll
    for (int i = 0; i < NAL; ++i) {
      const int row = ldr + RPL * i;
      if (row < tl.nrows)
        *reinterpret_cast<i32x4*>(Hout + (size_t)(tl.row0 + row) * ldh + it.nt * 128 + ldc * 16) =
            *reinterpret_cast<const i32x4*>(Hs + row * 128 + ldc * 16);
    }
    if (tid < FBM && tid < tl.nrows) {
      float am = amax_part[0][tid];
#pragma unroll
      for (int w = 1; w < NWN; ++w) am = fmaxf(am, amax_part[w][tid]);
      Sout[(size_t)(tl.row0 + tid) * (ldh / 128) + it.nt] = am > 0.f ? am / 448.0f : 1.0f;
    }
  }
}

bool wide_fp8_ok(const Dims& d) { return d.dtype == 2 && d.D % 128 == 0 && d.I % 128 == 0 && d.S % 128 == 0; }

hipError_t launch_wide_fp8(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s) {
  const int g0 = persistent_grid((const void*)gemm_wide_fp8<0>, 512) & ~7;
  const int g1 = persistent_grid((const void*)gemm_wide_fp8<1>, 256) & ~7;
  MOE_LAUNCH(gemm_wide_fp8<0>, dim3(g0), dim3(512), 0, s, (const uint8_t*)a.x, a.x_scale, nullptr, nullptr, nullptr,
             nullptr, a.row_token, a.offsets, a.tiles_wide, a.meta, (const uint8_t*)w.w1, (const uint8_t*)w.w3, w.s1,
             w.s3, (const uint8_t*)w.ws1, (const uint8_t*)w.ws3, w.ss1, w.ss3, a.h_routed, a.h_scale, a.h_shared,
             a.h_shared_scale, (int)d.T, d.D, d.I, d.S, d.E);
  MOE_LAUNCH(gemm_wide_fp8<1>, dim3(g1), dim3(256), 0, s, nullptr, nullptr, (const uint8_t*)a.h_routed, a.h_scale,
             (const uint8_t*)a.h_shared, a.h_shared_scale, a.row_token, a.offsets, a.tiles_wide, a.meta,
             (const uint8_t*)w.w2, nullptr, w.s2, nullptr, (const uint8_t*)w.ws2, nullptr, w.ss2, nullptr,
             a.o_routed, nullptr, a.o_shared, nullptr, (int)d.T, d.D, d.I, d.S, d.E);
  return hipGetLastError();
}

}  // namespace moe

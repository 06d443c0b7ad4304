// Prefill-sized expert GEMMs in bf16: M-tiles of 128 dispatch rows, LDS-staged operand
// tiles, 32x32x16 MFMA. The same SwiGLU expert as the 16-row kernels
// ("DeepSeek-V3.2-Exp · Mixture of experts": three dim x inter matrices per expert):
//   mode 0 (gate/up): h[rows, 64 cols] = silu(A W1^T) * (A W3^T), A = gathered x rows
//   mode 1 (down):    O[rows, 128 cols] = h W2^T
//
// Block: 256 threads = 4 waves in a 2 x 2 grid; block tile 128 rows x 128 weight rows
// (mode 0: 64 rows of W1 and the same 64 rows of W3, so each wave holds the gate and up
// accumulators of the same 32 h-columns), k-stage 64. Each stage is loaded from global
// memory into registers while the previous one is multiplied out of LDS. LDS rows are
// 128 bytes with their 16-byte chunks XOR-swizzled by row (swz), so both the stores and
// the MFMA fragment reads are free of bank conflicts.
//
// Work items are (expert, n-tile, m-tile) with the m-tiles of one weight tile adjacent,
// and a persistent grid hands each XCD (blockIdx % 8) a contiguous range of items, so the
// m-tiles that share a weight tile run together on one XCD and its L2 serves the re-reads.
#include "kernels.h"

namespace moe {

constexpr int WBM = kWideBM;  // 128 rows
constexpr int WBN = 128;      // weight rows per tile
constexpr int WBK = 64;       // k per stage: 128 bytes of bf16 per row
constexpr int kWideBlocksPerCU = 3;
constexpr int kWideGrid = 256 * kWideBlocksPerCU;

typedef __bf16 bf16x8w_t __attribute__((ext_vector_type(8)));

// D(32x32, fp32) += A(32x16) * B(16x32), bf16. Lane l holds A row / B column (l % 32) and eight
// consecutive k of chunk (l / 32); accumulator element 4j+i is row 8j + 4(l/32) + i, column l % 32.
MOE_DEV f32x16 mfma32(i32x4 a, i32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8w_t, a), __builtin_bit_cast(bf16x8w_t, b), c,
                                                 0, 0, 0);
}

template <int MODE>
__global__ __launch_bounds__(256, kWideBlocksPerCU) void gemm_wide_bf16(
    const bf16_t* __restrict__ act_x, const bf16_t* __restrict__ h_routed_in, const bf16_t* __restrict__ h_shared_in,
    const int32_t* __restrict__ row_token, const int32_t* __restrict__ offsets, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ meta, const bf16_t* __restrict__ wa, const bf16_t* __restrict__ wb,
    const bf16_t* __restrict__ wsa, const bf16_t* __restrict__ wsb, bf16_t* __restrict__ out_routed,
    bf16_t* __restrict__ out_shared, int T, int D, int I, int S, int E) {
  __shared__ __attribute__((aligned(16))) char smem[(WBM + WBN) * 128];
  char* As = smem;
  char* Bs = smem + WBM * 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;
  const int ldr = tid >> 3, ldc = tid & 7;  // this thread's load row (+32 i) and 16-byte chunk

  // n-tiles per expert: mode 0 covers 64 h-columns per tile, mode 1 128 output columns
  const int per_r = MODE == 0 ? I / 64 : D / 128;
  const int per_s = MODE == 0 ? S / 64 : D / 128;
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

    // global sources of this thread's 4 A rows and 4 B rows (row clamped into the tile)
    const bf16_t* asrc[4];
    const bf16_t* bsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = min(ldr + 32 * i, tl.nrows - 1);
      if (MODE == 0) {
        const int tok = sh ? tl.row0 + r : row_token[tl.row0 + r];
        asrc[i] = act_x + (size_t)tok * D + ldc * 8;
      } else {
        asrc[i] = (sh ? h_shared_in + (size_t)(tl.row0 + r) * S : h_routed_in + (size_t)(tl.row0 + r) * I) + ldc * 8;
      }
      const int br = ldr + 32 * i;  // 0..127
      if (MODE == 0) {
        const int hcol = it.nt * 64 + (br & 63);
        const bf16_t* W = br < 64 ? (sh ? wsa : wa + (size_t)tl.expert * I * D) : (sh ? wsb : wb + (size_t)tl.expert * I * D);
        bsrc[i] = W + (size_t)hcol * D + ldc * 8;
      } else {
        const bf16_t* W = sh ? wsa : wa + (size_t)tl.expert * D * I;
        bsrc[i] = W + (size_t)(it.nt * 128 + br) * K + ldc * 8;
      }
    }
    int lds_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_off[i] = swz(ldr + 32 * i, ldc);

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[a][b][q] = 0.f;

    i32x4 ra[4], rb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ld16(asrc[i]);
      rb[i] = ld16(bsrc[i]);
    }
    const int nk = K / WBK;
    for (int ks = 0; ks < nk; ++ks) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<i32x4*>(As + lds_off[i]) = ra[i];
        *reinterpret_cast<i32x4*>(Bs + lds_off[i]) = rb[i];
      }
      __syncthreads();
      if (ks + 1 < nk) {
        const int k = (ks + 1) * WBK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ra[i] = ld16(asrc[i] + k);
          rb[i] = ld16(bsrc[i] + k);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ch = kk * 2 + lh;
        i32x4 af[2], bfm[2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
          af[m] = *reinterpret_cast<const i32x4*>(As + swz(wm * 64 + m * 32 + l32, ch));
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int brow = MODE == 0 ? n * 64 + wn * 32 + l32 : wn * 64 + n * 32 + l32;
          bfm[n] = *reinterpret_cast<const i32x4*>(Bs + swz(brow, ch));
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int n = 0; n < 2; ++n) acc[m][n] = mfma32(af[m], bfm[n], acc[m][n]);
      }
    }

    // epilogue
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = wm * 64 + m * 32 + (q >> 2) * 8 + lh * 4 + (q & 3);
        if (row >= tl.nrows) continue;
        if (MODE == 0) {
          const float hv = silu_mul(acc[m][0][q], acc[m][1][q]);
          bf16_t* dst = sh ? out_shared + (size_t)(tl.row0 + row) * S : out_routed + (size_t)(tl.row0 + row) * I;
          dst[it.nt * 64 + wn * 32 + l32] = f32_to_bf16(hv);
        } else {
          bf16_t* dst = (sh ? out_shared : out_routed) + (size_t)(tl.row0 + row) * D + it.nt * 128 + wn * 64 + l32;
          dst[0] = f32_to_bf16(acc[m][0][q]);
          dst[32] = f32_to_bf16(acc[m][1][q]);
        }
      }
    }
  }
}

bool wide_ok(const Dims& d) { return d.dtype == 1 && d.D % 128 == 0 && d.I % 64 == 0 && d.S % 64 == 0; }

hipError_t launch_wide_bf16(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s) {
  if (wstream_ok(d)) return launch_wstream_bf16(d, w, a, s);
  if (ring_ok(d)) return launch_ring_bf16(d, w, a, s);
  MOE_LAUNCH(gemm_wide_bf16<0>, dim3(kWideGrid), dim3(256), 0, s, (const bf16_t*)a.x, nullptr, nullptr, a.row_token,
             a.offsets, a.tiles_wide, a.meta, (const bf16_t*)w.w1, (const bf16_t*)w.w3, (const bf16_t*)w.ws1,
             (const bf16_t*)w.ws3, (bf16_t*)a.h_routed, (bf16_t*)a.h_shared, (int)d.T, d.D, d.I, d.S, d.E);
  MOE_LAUNCH(gemm_wide_bf16<1>, dim3(kWideGrid), dim3(256), 0, s, nullptr, (const bf16_t*)a.h_routed,
             (const bf16_t*)a.h_shared, a.row_token, a.offsets, a.tiles_wide, a.meta, (const bf16_t*)w.w2, nullptr,
             (const bf16_t*)w.ws2, nullptr, (bf16_t*)a.o_routed, (bf16_t*)a.o_shared, (int)d.T, d.D, d.I, d.S, d.E);
  return hipGetLastError();
}

}  // namespace moe

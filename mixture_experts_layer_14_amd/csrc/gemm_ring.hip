// Prefill-sized bf16 expert GEMMs fed by a multi-stage ring of direct global->LDS loads.
// The SwiGLU expert of "DeepSeek-V3.2-Exp · Mixture of experts" (three dim x inter matrices):
//   mode 0 (gate/up): h = silu(A W1^T) * (A W3^T), A = gathered x rows
//   mode 1 (down):    O = h W2^T
//
// Block: 512 threads = 8 waves, one block per CU. Tile: BM rows x BN weight rows (mode 0:
// BN/2 rows of W1 and the same BN/2 rows of W3, so each wave holds the gate and up
// accumulators of the same h-columns), k-stage BK. STAGES stages live in LDS; STAGES - 1 are
// in flight while one is multiplied with 32x32x16 MFMAs, and one barrier per stage both
// publishes the landed stage and frees the slot the next load will fill.
//
// Partly filled M-tiles (most of them): activation rows past the tile's last row are not
// loaded (their load instructions are skipped and the wait counts follow), and waves whose
// 64 rows are all past it skip their MFMAs.
//
// Loads: global_load_lds_dwordx4 writes each wave instruction's 64 x 16 bytes to 1 KB of LDS;
// lane i loads the global 16-byte chunk that belongs at its slot under the XOR swizzle below,
// so operands never pass through registers and fragment reads are conflict-free. `s_waitcnt
// vmcnt` counts this wave's outstanding stage loads; a plain s_barrier (not __syncthreads,
// which would drain every load) publishes the stage.
//
// Items and the XCD-aware persistent grid are as in the other wide kernels.
#include "ring.h"

namespace moe {

constexpr int R_WAVES = 8;

typedef __bf16 bf16x8r_t __attribute__((ext_vector_type(8)));

MOE_DEV f32x16 mfma32r(i32x4 a, i32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8r_t, a), __builtin_bit_cast(bf16x8r_t, b), c,
                                                 0, 0, 0);
}

template <int MODE, int BM, int BN, int BK, int STAGES>
__global__ __launch_bounds__(64 * R_WAVES) void gemm_ring_bf16(
    const bf16_t* __restrict__ act_x, const bf16_t* __restrict__ h_routed_in, const bf16_t* __restrict__ h_shared_in,
    const int32_t* __restrict__ row_token, const int32_t* __restrict__ offsets, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ meta, const bf16_t* __restrict__ wa, const bf16_t* __restrict__ wb,
    const bf16_t* __restrict__ wsa, const bf16_t* __restrict__ wsb, bf16_t* __restrict__ out_routed,
    bf16_t* __restrict__ out_shared, int T, int D, int I, int S, int E) {
  constexpr int ROWB = BK * 2;           // bytes per LDS row
  constexpr int CPR = ROWB / 16;         // chunks per row
  constexpr int RPI = 64 / CPR;          // rows per load instruction
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB, STAGE = A_BYTES + B_BYTES;
  constexpr int A_INS = BM / RPI / R_WAVES, B_INS = BN / RPI / R_WAVES;
  constexpr int WM = BM / 64, WN = R_WAVES / WM;  // wave grid
  constexpr int NSUB = BN / WN / 32;              // 32-wide weight sub-tiles per wave
  constexpr int HN = MODE == 0 ? BN / 2 : BN;     // output columns per tile
  static_assert(A_INS >= 1 && B_INS >= 1 && WM * WN == R_WAVES && NSUB >= 1, "tile shape");
  static_assert(MODE == 1 || NSUB % 2 == 0, "gate/up pairs");
  extern __shared__ __attribute__((aligned(16))) char ring[];  // STAGES x STAGE bytes
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, lh = lane >> 5;
  const int lrow = lane / CPR, lpos = lane % CPR;  // row and slot of this lane in a load instruction

  const int per_r = MODE == 0 ? I / HN : D / HN;
  const int per_s = MODE == 0 ? S / HN : D / HN;
  const int nr = BM == kWideBM2 ? meta[5] : meta[2];
  const int items = nr * per_r + ((BM == kWideBM2 ? meta[6] : meta[3]) - nr) * per_s;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
  const int chunk = (items + 7) >> 3;

  for (int j = slot; j < chunk; j += per_xcd) {
    const int item = xcd * chunk + j;
    if (item >= items) break;
    const WideItem it = wide_item<BM>(item, tiles, nr, offsets, T, E, per_r, per_s);
    const Tile tl = it.tl;
    const bool sh = it.shared;
    const int K = MODE == 0 ? D : (sh ? S : I);

    // A load instructions of this wave that cover at least one real row, and their sources
    const bf16_t* asrc[A_INS];
    int na = 0;
#pragma unroll
    for (int q = 0; q < A_INS; ++q) {
      const int row = (wave * A_INS + q) * RPI + lrow;
      na += (wave * A_INS + q) * RPI < tl.nrows;
      const int r = min(row, tl.nrows - 1);
      const int c = lpos ^ ring_key<CPR>(row);
      if (MODE == 0) {
        const int tok = sh ? tl.row0 + r : row_token[tl.row0 + r];
        asrc[q] = act_x + (size_t)tok * D + c * 8;
      } else {
        asrc[q] = (sh ? h_shared_in + (size_t)(tl.row0 + r) * S : h_routed_in + (size_t)(tl.row0 + r) * I) + c * 8;
      }
    }
    const bf16_t* bsrc[B_INS];
#pragma unroll
    for (int q = 0; q < B_INS; ++q) {
      const int br = (wave * B_INS + q) * RPI + lrow;  // 0 .. BN-1
      const int c = lpos ^ ring_key<CPR>(br);
      if (MODE == 0) {
        const bf16_t* W = br < BN / 2 ? (sh ? wsa : wa + (size_t)tl.expert * I * D)
                                      : (sh ? wsb : wb + (size_t)tl.expert * I * D);
        bsrc[q] = W + (size_t)(it.nt * HN + br % (BN / 2)) * D + c * 8;
      } else {
        const bf16_t* W = sh ? wsa : wa + (size_t)tl.expert * D * I;
        bsrc[q] = W + (size_t)(it.nt * HN + br) * K + c * 8;
      }
    }
    const int per_stage = na + B_INS;  // load instructions this wave issues per stage
    auto issue = [&](int ks) {
      char* st = ring + (ks % STAGES) * STAGE;
      const int k = ks * BK;
#pragma unroll
      for (int q = 0; q < A_INS; ++q)
        if (q < na) lds_dma16(asrc[q] + k, st + (wave * A_INS + q) * 1024);
#pragma unroll
      for (int q = 0; q < B_INS; ++q) {
        // a weight tile read by this item only (its expert has one m-tile) is streamed nontemporally
        if (it.mt == 1)
          lds_dma16_nt(bsrc[q] + k, st + A_BYTES + (wave * B_INS + q) * 1024);
        else
          lds_dma16(bsrc[q] + k, st + A_BYTES + (wave * B_INS + q) * 1024);
      }
    };

    f32x16 acc[2][NSUB];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < NSUB; ++b)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[a][b][q] = 0.f;

    const int nk = K / BK;
    const bool active = wm * 64 < tl.nrows;  // this wave's 64 rows hold at least one row
    wait_vmcnt<0>();  // nothing else of this wave in flight: the counts below are exact
    __syncthreads();  // every wave is done with the ring of the previous item
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p)
      if (p < nk) issue(p);
    for (int ks = 0; ks < nk; ++ks) {
      // stages ks + 1 .. min(ks + STAGES - 2, nk - 1) may stay in flight
      wait_vmcnt_upto(min(STAGES - 2, nk - 1 - ks) * per_stage);
      barrier_only();  // stage ks landed for every wave; every wave is done with stage ks - 1
      if (ks + STAGES - 1 < nk) issue(ks + STAGES - 1);  // into the slot of stage ks - 1
      const char* As = ring + (ks % STAGES) * STAGE;
      const char* Bs = As + A_BYTES;
      if (active) {
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
          const int ch = kk * 2 + lh;
          i32x4 af[2], bfm[NSUB];
#pragma unroll
          for (int m = 0; m < 2; ++m)
            af[m] = *reinterpret_cast<const i32x4*>(As + ring_pos<CPR>(wm * 64 + m * 32 + l32, ch));
#pragma unroll
          for (int n = 0; n < NSUB; ++n) {
            // mode 0: the first NSUB/2 sub-tiles are gate rows, the rest the same h-columns of W3
            const int brow = MODE == 0 ? (n / (NSUB / 2)) * (BN / 2) + wn * (NSUB / 2) * 32 + (n % (NSUB / 2)) * 32 + l32
                                       : wn * NSUB * 32 + n * 32 + l32;
            bfm[n] = *reinterpret_cast<const i32x4*>(Bs + ring_pos<CPR>(brow, ch));
          }
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int n = 0; n < NSUB; ++n) acc[m][n] = mfma32r(af[m], bfm[n], acc[m][n]);
        }
      }
      wait_lgkm0();
    }

    if (active) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = wm * 64 + m * 32 + (q >> 2) * 8 + lh * 4 + (q & 3);
          if (row >= tl.nrows) continue;
          if (MODE == 0) {
            bf16_t* dst = (sh ? out_shared + (size_t)(tl.row0 + row) * S : out_routed + (size_t)(tl.row0 + row) * I) +
                          it.nt * HN + wn * (NSUB / 2) * 32 + l32;
#pragma unroll
            for (int n = 0; n < NSUB / 2; ++n)
              dst[n * 32] = f32_to_bf16(silu_mul(acc[m][n][q], acc[m][n + NSUB / 2][q]));
          } else {
            bf16_t* dst = (sh ? out_shared : out_routed) + (size_t)(tl.row0 + row) * D + it.nt * HN + wn * NSUB * 32 + l32;
#pragma unroll
            for (int n = 0; n < NSUB; ++n) dst[n * 32] = f32_to_bf16(acc[m][n][q]);
          }
        }
      }
    }
  }
}

// 256 x 256 tiles, 64-k stages, two stages in flight (128 KB of LDS)
constexpr int RBM = 256, RBN = 256, RBK = 64, RST = 2;

static size_t ring_lds() { return (size_t)RST * (RBM + RBN) * RBK * 2; }

bool ring_ok(const Dims& d) {
  const int lds_max = device_lds_limit();
  return d.dtype == 1 && ring_lds() <= (size_t)lds_max && d.D % RBN == 0 && d.I % (RBN / 2) == 0 &&
         d.S % (RBN / 2) == 0 && d.I % RBK == 0 && d.S % RBK == 0;
}

hipError_t launch_ring_bf16(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s) {
  const size_t lds = ring_lds();
  const void* k0 = (const void*)gemm_ring_bf16<0, RBM, RBN, RBK, RST>;
  const void* k1 = (const void*)gemm_ring_bf16<1, RBM, RBN, RBK, RST>;
  hipError_t attr = allow_dynamic_lds(k0, lds);
  if (attr == hipSuccess) attr = allow_dynamic_lds(k1, lds);
  if (attr != hipSuccess) return attr;  // never launch with more LDS than the kernel may take
  const Tile* tiles = RBM == kWideBM2 ? a.tiles_wide2 : a.tiles_wide;
  const int g0 = persistent_grid(k0, 64 * R_WAVES, lds) & ~7;
  const int g1 = persistent_grid(k1, 64 * R_WAVES, lds) & ~7;
  MOE_LAUNCH((gemm_ring_bf16<0, RBM, RBN, RBK, RST>), dim3(g0), dim3(64 * R_WAVES), lds, s, (const bf16_t*)a.x,
             nullptr, nullptr, a.row_token, a.offsets, tiles, a.meta, (const bf16_t*)w.w1, (const bf16_t*)w.w3,
             (const bf16_t*)w.ws1, (const bf16_t*)w.ws3, (bf16_t*)a.h_routed, (bf16_t*)a.h_shared, (int)d.T, d.D,
             d.I, d.S, d.E);
  MOE_LAUNCH((gemm_ring_bf16<1, RBM, RBN, RBK, RST>), dim3(g1), dim3(64 * R_WAVES), lds, s, nullptr,
             (const bf16_t*)a.h_routed, (const bf16_t*)a.h_shared, a.row_token, a.offsets, tiles, a.meta,
             (const bf16_t*)w.w2, nullptr, (const bf16_t*)w.ws2, nullptr, (bf16_t*)a.o_routed, (bf16_t*)a.o_shared,
             (int)d.T, d.D, d.I, d.S, d.E);
  return hipGetLastError();
}

}  // namespace moe

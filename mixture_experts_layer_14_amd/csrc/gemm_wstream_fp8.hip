// Prefill-sized FP8 (OCP e4m3fn) expert GEMMs with one weight stream per wave and fine-grained
// scales (weights: one fp32 scale per 128x128 block of the [out, in] matrix; activations: one per
// row per 128 columns). The SwiGLU expert of "DeepSeek-V3.2-Exp · Mixture of experts":
//   mode 0 (gate/up): h = silu(A W1^T) * (A W3^T), quantised per row per 128 columns in the
//                     epilogue (scale = amax / 448, 1 if amax = 0)
//   mode 1 (down):    O = h W2^T in bf16
//
// The weight-stream layout of the bf16 kernel with a step of one scale block (128 k = 128 bytes
// of every row): an item is an M-tile of up to 128 rows times 256 weight rows (mode 0: 128
// h-columns, their W1 rows and the W3 rows of the same columns, one 128-row scale block of each;
// mode 1: 256 output columns). 8 waves, two per SIMD, each multiply every row of the tile with
// their own 32 weight rows (mode 0: 16 W1 rows over the W3 rows of the same columns, so a lane
// holds gate and up of its h-values). Both operands and the tile's row scales go global -> LDS
// directly (buffer loads with an LDS destination): three stages of activations + row scales
// shared by the block, three weight slabs per wave, both two steps ahead of the MFMAs.
//
// A step's partial products come from two 32x32x64 fp8 MFMAs started from zero per 32 x 32 tile;
// they are added to the fp32 accumulators times sx(row) * sw, sw being the weight scale of the
// step's block. Both scales reach LDS with the stage (the row scales through waves 0-3's 4-byte
// loads, the step's weight scales through waves 4 and 5's), so the loop has no scalar memory
// loads: a scalar load shares the LDS wait counter, and waiting for it stalled every step on the
// scalar cache and drained the fragment reads in flight. The MFMAs take the weights as their first operand, so the 16
// elements of a lane belong to one activation row and share sx: a promotion costs one product per
// scale and one FMA per element, and the other wave of the SIMD issues MFMAs meanwhile.
//
// Step n: wait until this wave's part of stage n and its slab n have landed, barrier (stage n is
// complete and every wave is done with stage n - 1), multiply, and request stage and slab n + 2
// one or two loads after each row group's MFMAs (issued in one burst before the MFMAs, the loads
// held them up: 13% slower). Loads complete in issue order, so activations, row scales and weights
// of a step all go out within the step and the wait at step n leaves stage and slab n + 1 in
// flight. The step sequence runs on across the block's items; steps come in groups of four, so
// dim / 128 and inter / 128 must be multiples of four.
#include <type_traits>

#include "wstream.h"

namespace moe {

constexpr int WQ_WAVES = 8;
constexpr int WQ_BM = kWideBM;                                   // rows per M-tile (128)
constexpr int WQ_NS = 3;                                         // stages and slabs per wave
constexpr int WQ_A = WQ_BM * 128;                                // 16 KB per activation stage
constexpr int WQ_SX = WQ_WAVES * 256;                            // scales: wave w's 64 lanes x 4 B
constexpr int WQ_SLAB = 32 * 128;                                // 4 KB per weight slab
constexpr int WQ_AQ = WQ_BM / 8 / WQ_WAVES;                      // activation loads per wave and step (2)
constexpr int WQ_BQ = 4;                                         // weight loads per wave and step
constexpr int WQ_NM = WQ_BM / 32;                                // 32-row groups of a tile
constexpr int WQ_SX0 = WQ_NS * WQ_A;                             // LDS offsets
constexpr int WQ_B0 = WQ_SX0 + WQ_NS * WQ_SX;
constexpr int WQ_AM = WQ_B0 + WQ_WAVES * WQ_NS * WQ_SLAB;        // amax exchange: 8 waves x 128 rows
constexpr size_t WQ_LDS = (size_t)WQ_AM + (size_t)WQ_WAVES * WQ_BM * 4;  // 154 KB

// D(32x32, fp32) += A(32x64) * B(64x32), e4m3 codes with unit block scales (E8M0 127 = 1.0).
// Lane l holds A row / B column (l % 32) and 32 consecutive k of half (l / 32).
MOE_DEV f32x16 mfma32q(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

MOE_DEV i32x8 ws_frag32(const char* base, int off_lo, int off_hi) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(base + off_lo);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(base + off_hi);
  i32x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return r;
}

template <int MODE>
__global__ __launch_bounds__(64 * WQ_WAVES) void gemm_wstream_fp8(
    const uint8_t* __restrict__ aq, const float* __restrict__ a_scale,  // mode 0: xq [T, D], sx [T, D/128]
    const uint8_t* __restrict__ h_routed_in, const float* __restrict__ hs_routed_in,
    const uint8_t* __restrict__ h_shared_in, const float* __restrict__ hs_shared_in,
    const int32_t* __restrict__ row_token, const int32_t* __restrict__ offsets, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ meta, const uint8_t* __restrict__ wa, const uint8_t* __restrict__ wb,
    const float* __restrict__ sa, const float* __restrict__ sb_, const uint8_t* __restrict__ wsa,
    const uint8_t* __restrict__ wsb, const float* __restrict__ ssa, const float* __restrict__ ssb,
    void* __restrict__ out_routed, float* __restrict__ outs_routed, void* __restrict__ out_shared,
    float* __restrict__ outs_shared, int T, int D, int I, int S, int E) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, lh = lane >> 5;
  constexpr int HN = MODE == 0 ? 128 : 256;  // output columns per item
  const int per_r = MODE == 0 ? I / HN : D / HN;
  const int per_s = MODE == 0 ? S / HN : D / HN;
  const int nr = meta[2];
  const int items = nr * per_r + (meta[3] - nr) * per_s;
  // this block's items: xcd * chunk + slot + i * per_xcd for i < mine (an XCD's blocks share a range)
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
  // gate/up: each XCD's range starts at a multiple of per_r items (one tile's column items), so the
  // blocks that take a round's consecutive items cover whole tiles (16 of them per tile for inter
  // 2048: half of an XCD's 32 blocks) and share its activation rows
  const int chunk = MODE == 0 ? (((items + 7) >> 3) + per_r - 1) / per_r * per_r : (items + 7) >> 3;
  const int lim = min(chunk, items - xcd * chunk);
  const int mine = slot < lim ? (lim - slot + per_xcd - 1) / per_xcd : 0;
  if (mine == 0) return;
  const int nk = (MODE == 0 ? D : I) / 128;  // steps (scale blocks) per item; the shared expert has S == I

  auto item_of = [&](int i) __attribute__((always_inline)) {
    WsItem d;
    d.live = i < mine;
    d.row0 = 0, d.nrows = 0, d.nt = 0, d.expert = 0, d.rot = 0, d.sh = false, d.solo = false;
    if (d.live) {
      const WideItem it = wide_item<WQ_BM>(xcd * chunk + slot + i * per_xcd, tiles, nr, offsets, T, E, per_r, per_s);
      d.row0 = it.tl.row0;
      d.nrows = it.tl.nrows;
      d.nt = it.nt;
      d.expert = it.tl.expert;
      d.sh = it.shared;
      // each item starts its k walk at its own block, so concurrent items spread over the HBM channels
      d.rot = (MODE == 0 ? 3 * d.expert : 3 * d.expert + 5 * d.nt) % nk;
    }
    return d;
  };
  auto blk = [&](int ks, int rot) __attribute__((always_inline)) {  // scale block of step ks
    int s = ks + rot;
    if (s >= nk) s -= nk;
    return s;
  };
  // the lane index as a value the compiler cannot hoist (see the bf16 kernel)
  auto lane_now = [&]() __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    return ln;
  };

  // ---- weight stream of this wave: 32 rows, 128 bytes of each per step; instruction i covers
  // slab rows 8 i .. 8 i + 7 (mode 0: W1 rows of the wave's 16 h-columns for i < 2, the W3 rows of
  // the same columns after). A lane's source chunk makes slab row r's chunk c land in 16-byte slot
  // c ^ ws_key(r); ws_key(8 i + lane / 8) = lane / 8 ^ i.
  __amdgpu_buffer_rsrc_t br0, br1;
  int b_row8, b_rot, b_voff[WQ_BQ];
  auto b_set = [&](const WsItem& d) __attribute__((always_inline)) {
    int ldb;
    if (MODE == 0) {
      const size_t r = (size_t)d.nt * HN + wave * 16;
      br0 = ws_rsrc((d.sh ? wsa : wa + (size_t)d.expert * I * D) + r * D, 16 * D);
      br1 = ws_rsrc((d.sh ? wsb : wb + (size_t)d.expert * I * D) + r * D, 16 * D);
      ldb = D;
    } else {
      br0 = ws_rsrc((d.sh ? wsa : wa + (size_t)d.expert * D * I) + ((size_t)d.nt * HN + wave * 32) * I, 32 * I);
      br1 = br0;
      ldb = I;
    }
    b_row8 = __builtin_amdgcn_readfirstlane(8 * ldb);
    b_rot = d.rot;
    const int ln = lane_now();
#pragma unroll
    for (int i = 0; i < WQ_BQ; ++i)
      b_voff[i] = d.live ? (ln >> 3) * ldb + ((((ln & 7) ^ (ln >> 3)) ^ i) << 4) : WS_OOB;
  };
  char* const wslab = lds + WQ_B0 + wave * (WQ_NS * WQ_SLAB);  // this wave's three slabs
  // instructions I0 .. I1 - 1 of the slab
  auto issue_b = [&](auto i0, auto i1, int slot_b, int ks) __attribute__((always_inline)) {
    constexpr int I0 = decltype(i0)::value, I1 = decltype(i1)::value;
    const int kb = blk(ks, b_rot) * 128;
    char* dst = wslab + slot_b * WQ_SLAB;
#pragma unroll
    for (int i = I0; i < I1; ++i)
      ws_dma<false>(MODE == 0 && i >= 2 ? br1 : br0, dst + i * 1024, b_voff[i],
                    kb + (MODE == 0 ? (i & 1) : i) * b_row8);
  };

  // ---- activation rows: instruction q of wave w fills tile rows 16 w + 8 q + lane / 8; row
  // scales: waves 0..3 fill rows 32 w + lane (lanes < 32) into their own 256 bytes, the other
  // waves' areas get zeros. Mode 0 needs tokens: lane l < 32 holds the token of row
  // 32 (w % 4) + l, lane l >= 32 that of row 16 w + l % 16 (rows clamped to the tile), loaded a
  // step before a_set needs them so that waiting for them does not drain the loads in flight.
  auto tok_load = [&](const WsItem& d) __attribute__((always_inline)) {
    int t = 0;
    if (MODE == 0 && d.live) {
      const int ln = lane_now();
      const int r = min(ln < 32 ? (wave & 3) * 32 + ln : wave * 16 + (ln & 15), d.nrows - 1);
      t = d.sh ? d.row0 + r : row_token[d.row0 + r];
    }
    return t;
  };
  const uint8_t* a_base;
  const float* s_base;
  int a_voff[WQ_AQ], s_voff, a_rot;
  auto a_set = [&](const WsItem& d, int tok_mine) __attribute__((always_inline)) {
    const int ln = lane_now();
    a_base = MODE == 0 ? aq : (d.sh ? h_shared_in : h_routed_in);
    a_rot = d.rot;
    const int row_bytes = MODE == 0 ? D : (d.sh ? S : I);
#pragma unroll
    for (int q = 0; q < WQ_AQ; ++q) {
      const int a_row = wave * 16 + q * 8 + (ln >> 3);  // tile row; its key is lane / 8 ^ (2 w + q) % 4
      const int c16 = (((ln & 7) ^ (ln >> 3)) ^ ((2 * wave + q) & 3)) << 4;
      int off = WS_OOB;
      if (MODE == 0) {
        const int tok = __shfl(tok_mine, 32 + q * 8 + (ln >> 3));
        if (d.live && a_row < d.nrows) off = tok * row_bytes + c16;
      } else {
        if (d.live && a_row < d.nrows) off = (d.row0 + a_row) * row_bytes + c16;
      }
      a_voff[q] = off;
    }
    const int s_row = wave * 32 + ln;
    const int tok_s = MODE == 0 ? tok_mine : d.row0 + s_row;
    if (wave < 4) {  // the tile rows' scales
      s_base = MODE == 0 ? a_scale : (d.sh ? hs_shared_in : hs_routed_in);
      s_voff = (d.live && ln < 32 && s_row < d.nrows) ? tok_s * (nk * 4) : WS_OOB;
    } else {  // the weight scale of the step's block: waves 4 and 5, lane 0
      if (MODE == 0) {  // wave 4: W1's 128x128 block row holding the item's h-columns, wave 5: W3's
        const size_t nb = I / 128;
        s_base = (wave == 4 ? (d.sh ? ssa : sa + (size_t)d.expert * nb * nk)
                            : (d.sh ? ssb : sb_ + (size_t)d.expert * nb * nk)) + (size_t)d.nt * nk;
      } else {  // wave 4: the W2 block row of waves 0-3's output columns, wave 5: that of waves 4-7
        const size_t nb = D / 128;
        s_base = (d.sh ? ssa : sa + (size_t)d.expert * nb * nk) + (size_t)(d.nt * 2 + (wave & 1)) * nk;
      }
      s_voff = (d.live && wave < 6 && ln == 0) ? 0 : WS_OOB;
    }
  };
  auto issue_a = [&](int stage, int ks) __attribute__((always_inline)) {
    const int kbi = blk(ks, a_rot);
    const __amdgpu_buffer_rsrc_t r = ws_rsrc(a_base, WS_RANGE);
    char* dst = lds + stage * WQ_A + wave * WQ_AQ * 1024;
#pragma unroll
    for (int q = 0; q < WQ_AQ; ++q) ws_dma<false>(r, dst + q * 1024, a_voff[q], kbi * 128);
  };
  auto issue_s = [&](int stage, int ks) __attribute__((always_inline)) {  // the stage's row and weight scales
    const int kbi = blk(ks, a_rot);
    const __amdgpu_buffer_rsrc_t rs = ws_rsrc(s_base, WS_RANGE);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(lds + WQ_SX0 + stage * WQ_SX + wave * 256), 4, s_voff, kbi * 4, 0,
        0);
  };

  // ---- one step: acc[m] += (W(wave rows) A(tile rows 32 m ..)^T) * scales; element q of a lane is
  // weight row 8 (q / 4) + 4 lh + q % 4 of the wave (mode 0: q < 8 gate, q >= 8 up of the same
  // column) and tile row 32 m + l32
  f32x16 acc[WQ_NM];
  // fragment offsets: 64-k half kk, 16-byte half h: chunk 4 kk + 2 lh + h of row l32
  int foff[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h) foff[kk][h] = ws_pos(l32, kk * 4 + lh * 2 + h);
  const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // issue(m) runs after the MFMAs of row group m: the step's loads go out between its MFMAs
  // instead of in one burst before them.
  auto compute = [&](int st, auto&& issue) __attribute__((always_inline)) {
    const char* As = lds + st * WQ_A;
    const char* Bs = wslab + st * WQ_SLAB;
    // tile row 32 m + l32's scale: wave m's area holds rows 32 m .. 32 m + 31; the weight scales
    // are the first word of waves 4 and 5's areas (mode 1: the one of this wave's half)
    const float* sxa = reinterpret_cast<const float*>(lds + WQ_SX0 + st * WQ_SX);
    const float* sxs = sxa + l32;
    const float sw0 = sxa[(MODE == 0 ? 4 : 4 + (wave >> 2)) * 64];
    const float sw1 = MODE == 0 ? sxa[5 * 64] : sw0;
    const i32x8 b0 = ws_frag32(Bs, foff[0][0], foff[0][1]);
    const i32x8 b1 = ws_frag32(Bs, foff[1][0], foff[1][1]);
    i32x8 a0 = ws_frag32(As, foff[0][0], foff[0][1]);
    i32x8 a1 = ws_frag32(As, foff[1][0], foff[1][1]);
    float sx = sxs[0], sx_prev = 0.f;
    f32x16 p[2];
    auto promote = [&](int m, const f32x16& pm, float s) __attribute__((always_inline)) {
      const float f0 = s * sw0, f1 = MODE == 0 ? s * sw1 : f0;
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[m][q] += pm[q] * (q < 8 ? f0 : f1);
    };
#pragma unroll
    for (int m = 0; m < WQ_NM; ++m) {
      p[m & 1] = mfma32q(b1, a1, mfma32q(b0, a0, zero16));
      issue(m);
      const float sx_m = sx;
      if (m + 1 < WQ_NM) {  // next group's rows and scale; read after the MFMAs that use a0 / a1
        a0 = ws_frag32(As + (m + 1) * 4096, foff[0][0], foff[0][1]);
        a1 = ws_frag32(As + (m + 1) * 4096, foff[1][0], foff[1][1]);
        sx = sxs[(m + 1) * 64];
      }
      if (m > 0) promote(m - 1, p[(m - 1) & 1], sx_prev);
      sx_prev = sx_m;
      __builtin_amdgcn_sched_barrier(0);  // keeps the group's reads from being hoisted (registers)
    }
    promote(WQ_NM - 1, p[(WQ_NM - 1) & 1], sx_prev);
  };
  // ---- epilogues. A lane holds tile row 32 m + l32 and, for each jj = q / 4, the four
  // consecutive weight rows 8 jj + 4 lh .. + 3 of the wave, stored as one 4-byte word (mode 0:
  // codes of h-columns 16 wave + 8 jj + 4 lh ..) or 8-byte word (mode 1: bf16 of output columns
  // 32 wave + 8 jj + 4 lh ..). Stores go through buffer resources spanning the item's rows, so rows
  // past its end are dropped.
  float* amax_part = reinterpret_cast<float*>(lds + WQ_AM);  // [wave][128 rows]
  auto epilogue = [&](const WsItem& d) __attribute__((always_inline)) {
    const int ln = lane_now();
    const int lo32 = ln & 31, lhi = ln >> 5;
    if (MODE == 0) {
      // h = silu(g) * u in place; per row amax over the wave's 16 h-columns, then over the waves
      const int ld = d.sh ? S : I;
#pragma unroll
      for (int m = 0; m < WQ_NM; ++m) {
        float a = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          acc[m][q] = silu_mul(acc[m][q], acc[m][q + 8]);
          a = fmaxf(a, fabsf(acc[m][q]));
        }
        a = fmaxf(a, __shfl_xor(a, 32));
        if (lhi == 0) amax_part[wave * WQ_BM + m * 32 + lo32] = a;
      }
      __syncthreads();
      const __amdgpu_buffer_rsrc_t o = ws_rsrc(static_cast<uint8_t*>(d.sh ? out_shared : out_routed) + (size_t)d.row0 * ld,
                                               d.nrows * ld);
      const __amdgpu_buffer_rsrc_t os = ws_rsrc((d.sh ? outs_shared : outs_routed) + (size_t)d.row0 * (ld / 128),
                                                d.nrows * (ld / 128) * 4);
#pragma unroll
      for (int m = 0; m < WQ_NM; ++m) {
        const int row = m * 32 + lo32;
        float am = amax_part[row];
#pragma unroll
        for (int w = 1; w < WQ_WAVES; ++w) am = fmaxf(am, amax_part[w * WQ_BM + row]);
        const float scale = am > 0.f ? am / 448.0f : 1.0f;
        const int vrow = row * ld + d.nt * 128 + wave * 16 + lhi * 4;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const uint32_t c = f32x2_to_e4m3(acc[m][jj * 4] / scale, acc[m][jj * 4 + 1] / scale) |
                             (f32x2_to_e4m3(acc[m][jj * 4 + 2] / scale, acc[m][jj * 4 + 3] / scale) << 16);
          __builtin_amdgcn_raw_buffer_store_b32(c, o, vrow + jj * 8, 0, 0);
        }
        if (wave == 0 && lhi == 0)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(scale), os, (row * (ld / 128) + d.nt) * 4, 0, 0);
      }
    } else {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const __amdgpu_buffer_rsrc_t o = ws_rsrc(static_cast<bf16_t*>(d.sh ? out_shared : out_routed) + (size_t)d.row0 * D,
                                               d.nrows * D * 2);
#pragma unroll
      for (int m = 0; m < WQ_NM; ++m) {
        const int vrow = ((m * 32 + lo32) * D + d.nt * HN + wave * 32 + lhi * 4) * 2;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const u32x2 w = {(uint32_t)f32_to_bf16(acc[m][jj * 4]) | ((uint32_t)f32_to_bf16(acc[m][jj * 4 + 1]) << 16),
                           (uint32_t)f32_to_bf16(acc[m][jj * 4 + 2]) | ((uint32_t)f32_to_bf16(acc[m][jj * 4 + 3]) << 16)};
          __builtin_amdgcn_raw_buffer_store_b64(w, o, vrow + jj * 16, 0, 0);
        }
      }
    }
  };

  // Step n of the item, stage and slab of step n in slot st: request stage and slab n + 2 (at
  // step ks of the load cursor's item) and multiply.
  int st = 0;
  auto step = [&](int ks, int ks_c) __attribute__((always_inline)) {
    (void)ks_c;
    wait_vmcnt<WQ_AQ + 1 + WQ_BQ>();  // loads after slab n: stage n + 1 (+ its scales), slab n + 1
    wait_lgkm0();
    barrier_only();
    const int s2 = st == 0 ? 2 : st - 1;
    compute(st, [&](int m) __attribute__((always_inline)) {
      using std::integral_constant;
      if (m == 0) issue_a(s2, ks);
      if (m == 1) {
        issue_s(s2, ks);
        issue_b(integral_constant<int, 0>{}, integral_constant<int, 1>{}, s2, ks);
      }
      if (m == 2) issue_b(integral_constant<int, 1>{}, integral_constant<int, 3>{}, s2, ks);
      if (m == 3) issue_b(integral_constant<int, 3>{}, integral_constant<int, WQ_BQ>{}, s2, ks);
    });
    st = st == 2 ? 0 : st + 1;
  };
  auto body = [&]() __attribute__((always_inline)) {
    for (int g = 0; g < nk / 4 - 1; ++g) {
      const int k0 = 4 * g;
      step(k0 + 2, k0);
      step(k0 + 3, k0 + 1);
      step(k0 + 4, k0 + 2);
      step(k0 + 5, k0 + 3);
    }
  };
  // the final group: the load cursor moves to the next item after the second step
  auto tail = [&](const WsItem& next) __attribute__((always_inline)) {
    const int tok_next = tok_load(next);
    step(nk - 2, nk - 4);
    step(nk - 1, nk - 3);
    a_set(next, tok_next);
    b_set(next);
    step(0, nk - 2);
    step(1, nk - 1);
  };

  // prologue, in the issue order of the steps before step 0: stage and slab 0, then 1
  WsItem cur = item_of(0);
  b_set(cur);
  a_set(cur, tok_load(cur));
  wait_vmcnt<0>();
  using std::integral_constant;
  issue_a(0, 0);
  issue_s(0, 0);
  issue_b(integral_constant<int, 0>{}, integral_constant<int, WQ_BQ>{}, 0, 0);
  issue_a(1, 1);
  issue_s(1, 1);
  issue_b(integral_constant<int, 0>{}, integral_constant<int, WQ_BQ>{}, 1, 1);

  for (int i = 0; i < mine; ++i) {
#pragma unroll
    for (int m = 0; m < WQ_NM; ++m)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[m][q] = 0.f;
    const WsItem next = item_of(i + 1);
    body();
    tail(next);
    // the accumulators are final here: keeps the compiler from sinking the tail's MFMAs into the
    // epilogue, where the operands they read would have to be kept (spilled) until then
#pragma unroll
    for (int m = 0; m < WQ_NM; ++m) asm volatile("" : "+v"(acc[m]));
    epilogue(cur);
    cur = next;
  }
  wait_vmcnt<0>();  // no LDS write may still be in flight when the block ends
}

bool wstream_fp8_ok(const Dims& d) {
  const int lds_max = device_lds_limit();
  const int64_t lim = WS_RANGE - (1 << 20);
  return d.dtype == 2 && WQ_LDS <= (size_t)lds_max && d.D % 512 == 0 && d.I % 512 == 0 && d.S == d.I &&
         d.T * d.D < lim && d.R * d.I < lim && d.T * d.S < lim && d.R * (d.I / 128) * 4 < lim &&
         d.T * (d.D / 128) * 4 < lim;
}

hipError_t launch_wstream_fp8(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s) {
  const void* k0 = (const void*)gemm_wstream_fp8<0>;
  const void* k1 = (const void*)gemm_wstream_fp8<1>;
  hipError_t attr = allow_dynamic_lds(k0, WQ_LDS);
  if (attr == hipSuccess) attr = allow_dynamic_lds(k1, WQ_LDS);
  if (attr != hipSuccess) return attr;  // never launch with more LDS than the kernel may take
  const int g0 = persistent_grid(k0, 64 * WQ_WAVES, WQ_LDS) & ~7;
  const int g1 = persistent_grid(k1, 64 * WQ_WAVES, WQ_LDS) & ~7;
  MOE_LAUNCH(gemm_wstream_fp8<0>, dim3(g0), dim3(64 * WQ_WAVES), WQ_LDS, s, (const uint8_t*)a.x, a.x_scale, nullptr,
             nullptr, nullptr, nullptr, a.row_token, a.offsets, a.tiles_wide, a.meta, (const uint8_t*)w.w1,
             (const uint8_t*)w.w3, w.s1, w.s3, (const uint8_t*)w.ws1, (const uint8_t*)w.ws3, w.ss1, w.ss3, a.h_routed,
             a.h_scale, a.h_shared, a.h_shared_scale, (int)d.T, d.D, d.I, d.S, d.E);
  MOE_LAUNCH(gemm_wstream_fp8<1>, dim3(g1), dim3(64 * WQ_WAVES), WQ_LDS, s, nullptr, nullptr,
             (const uint8_t*)a.h_routed, a.h_scale, (const uint8_t*)a.h_shared, a.h_shared_scale, a.row_token,
             a.offsets, a.tiles_wide, a.meta, (const uint8_t*)w.w2, nullptr, w.s2, nullptr, (const uint8_t*)w.ws2,
             nullptr, w.ss2, nullptr, a.o_routed, nullptr, a.o_shared, nullptr, (int)d.T, d.D, d.I, d.S, d.E);
  return hipGetLastError();
}

}  // namespace moe

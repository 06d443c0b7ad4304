// Prefill-sized bf16 expert GEMMs with one weight stream per wave.
// The SwiGLU expert of "DeepSeek-V3.2-Exp · Mixture of experts" (three dim x inter matrices):
//   mode 0 (gate/up): h = silu(A W1^T) * (A W3^T), A = gathered x rows
//   mode 1 (down):    O = h W2^T
//
// Item: an M-tile of up to 128 rows of one expert times 256 weight rows (mode 0: 128
// h-columns, i.e. their W1 rows and the W3 rows of the same columns; mode 1: 256 output
// columns). Block: 4 waves, one block per CU (one wave per SIMD). Every wave multiplies all rows
// of the M-tile with its own 64 weight rows (mode 0: 32 W1 rows and the 32 matching W3 rows, so
// gate and up of one h-column meet in one lane), so no wave idles on a partly filled tile.
//
// Both operands go from global memory straight into LDS (buffer loads with an LDS destination;
// each lane fetches the 16-byte chunk that belongs at its slot under the swizzle below):
//   weights, read once from HBM: a wave-private ring of three 64-k slabs (64 rows x 128 bytes; one
//     instruction reads 8 rows x 128 contiguous bytes), two slabs in flight while the third is
//     multiplied: 64 KB of weights in flight per CU. The weight loads of an expert with a single
//     M-tile are nontemporal (no other item reads those tiles), and so are all weight loads when
//     the routed experts average less than one M-tile.
//   activation rows (small, L2-resident): a 4-stage ring shared by the block; rows past the
//     tile's end take an out-of-range offset and read as zeros without touching memory.
//
// Step n (64 k of one item): wait until this wave's part of activation stage n and its slab n
// have landed, barrier (stage n is complete and every wave is done with stage n - 1), multiply,
// and request slab n + 2 and activation stage n + 3 between the MFMAs of the step's four k-steps
// (issued in one burst before them, the twelve loads held up the MFMAs: 3% slower). Vector-memory
// loads complete in issue order; each step issues its weight loads (HBM latency) before its
// activation loads (L2 hits, needed three steps later), so the wait at step n leaves stage n + 1,
// slab n + 1 and stage n + 2 in flight (activations first measured 1-2% slower). The step sequence runs on across the block's items without draining: an item's last
// steps request the next item's first stages. A ragged tile multiplies only its live 32-row groups.
//
// Steps come in groups of four (the activation stages rotate with the group), so an item's steps
// (dim / 64 or inter / 64) must be a multiple of four; the epilogue and the accumulator reset run
// between items, outside the unrolled group. Every wait above is an explicit count: all loads of
// the loop are LDS-destination loads, which the compiler neither reorders nor waits for itself.
#include <type_traits>

#include "wstream.h"

namespace moe {

constexpr int WS_WAVES = 4;
constexpr int WS_WROWS = 64;                                         // weight rows per wave
constexpr int WS_BM = kWideBM;                                       // rows per M-tile (128)
constexpr int WS_BK = 64;                                            // k per step
constexpr int WS_NA = 4;                                             // activation stages
constexpr int WS_NB = 3;                                             // weight slabs per wave
constexpr int WS_A_STAGE = WS_BM * WS_BK * 2;                        // 16 KB
constexpr int WS_SLAB = WS_WROWS * WS_BK * 2;                        // 8 KB
constexpr int WS_AQ = WS_BM / 8 / WS_WAVES;                          // activation loads per wave and step
constexpr int WS_BQ = WS_WROWS / 8;                                  // weight loads per wave and step
constexpr int WS_NM = WS_BM / 32;                                    // 32-row groups of an M-tile
constexpr int WS_B0 = WS_NA * WS_A_STAGE;                            // LDS offset of the slabs
constexpr size_t WS_LDS = (size_t)WS_B0 + (size_t)WS_WAVES * WS_NB * WS_SLAB;  // 160 KB

typedef __bf16 bf16x8w_t __attribute__((ext_vector_type(8)));

MOE_DEV f32x16 mfma32w(i32x4 a, i32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8w_t, a), __builtin_bit_cast(bf16x8w_t, b), c,
                                                 0, 0, 0);
}

// NT: every weight load nontemporal (else only the tiles of single-M-tile experts)
template <int MODE, bool NT>
__global__ __launch_bounds__(64 * WS_WAVES) void gemm_wstream_bf16(
    const bf16_t* __restrict__ act_x, const bf16_t* __restrict__ h_routed_in, const bf16_t* __restrict__ h_shared_in,
    const int32_t* __restrict__ row_token, const int32_t* __restrict__ offsets, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ meta, const bf16_t* __restrict__ wa, const bf16_t* __restrict__ wb,
    const bf16_t* __restrict__ wsa, const bf16_t* __restrict__ wsb, bf16_t* __restrict__ out_routed,
    bf16_t* __restrict__ out_shared, int T, int D, int I, int S, int E) {
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
  const int chunk = (items + 7) >> 3;
  const int lim = min(chunk, items - xcd * chunk);
  const int mine = slot < lim ? (lim - slot + per_xcd - 1) / per_xcd : 0;
  if (mine == 0) return;
  const int nk = (MODE == 0 ? D : I) / WS_BK;  // steps per item (the shared expert has S == I)

  auto item_of = [&](int i) __attribute__((always_inline)) {
    WsItem d;
    d.live = i < mine;
    d.row0 = 0, d.nrows = 0, d.nt = 0, d.expert = 0, d.rot = 0, d.sh = false, d.solo = false;
    if (d.live) {
      const WideItem it = wide_item<WS_BM>(xcd * chunk + slot + i * per_xcd, tiles, nr, offsets, T, E, per_r, per_s);
      d.row0 = it.tl.row0;
      d.nrows = it.tl.nrows;
      d.nt = it.nt;
      d.expert = it.tl.expert;
      d.sh = it.shared;
      d.solo = it.mt == 1;
      // each item starts its k walk at its own step, so concurrent items spread over the HBM channels
      d.rot = (MODE == 0 ? 3 * d.expert : 3 * d.expert + 5 * d.nt) % nk;
    }
    return d;
  };
  auto kbytes = [&](int ks, int rot) __attribute__((always_inline)) {
    int s = ks + rot;
    if (s >= nk) s -= nk;
    return s * (WS_BK * 2);
  };
  // the lane index as a value the compiler cannot hoist: lane-derived values of the rarely run
  // item set-up code are recomputed there instead of occupying registers across the step loop
  auto lane_now = [&]() __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    return ln;
  };

  // ---- weight stream of this wave: 64 rows, 128 bytes of each per step; instruction i covers
  // slab rows 8 i .. 8 i + 7 (mode 0: W1 rows for i < 4, the W3 rows of the same columns after)
  __amdgpu_buffer_rsrc_t br0, br1;
  int b_row8, b_rot, b_voff[4];
  bool b_solo = false;
  auto b_set = [&](const WsItem& d) __attribute__((always_inline)) {
    int ldb;
    if (MODE == 0) {
      const size_t r = (size_t)d.nt * HN + wave * 32;
      br0 = ws_rsrc((d.sh ? wsa : wa + (size_t)d.expert * I * D) + r * D, 32 * D * 2);
      br1 = ws_rsrc((d.sh ? wsb : wb + (size_t)d.expert * I * D) + r * D, 32 * D * 2);
      ldb = D * 2;
    } else {
      br0 = ws_rsrc((d.sh ? wsa : wa + (size_t)d.expert * D * I) + ((size_t)d.nt * HN + wave * 64) * I, 64 * I * 2);
      br1 = br0;
      ldb = I * 2;
    }
    b_row8 = __builtin_amdgcn_readfirstlane(8 * ldb);
    b_rot = d.rot;
    b_solo = d.solo;
    const int ln = lane_now();
#pragma unroll
    for (int i = 0; i < 4; ++i)
      b_voff[i] = d.live ? (ln >> 3) * ldb + ((((ln & 7) ^ (ln >> 3)) ^ i) << 4) : WS_OOB;
  };
  char* const wslab = lds + WS_B0 + wave * (WS_NB * WS_SLAB);  // this wave's three slabs
  // instructions I0 .. I1 - 1 of the slab
  auto issue_b = [&](auto i0, auto i1, int slot_b, int ks) __attribute__((always_inline)) {
    constexpr int I0 = decltype(i0)::value, I1 = decltype(i1)::value;
    const int kb = kbytes(ks, b_rot);
    char* dst = wslab + slot_b * WS_SLAB;
    // weight tiles of a single-M-tile expert are read by one item only: nontemporal, so they do not
    // push out of L2 the tiles that other M-tiles of an expert are about to read
    if (b_solo) {
#pragma unroll
      for (int i = I0; i < I1; ++i)
        ws_dma<true>(MODE == 0 && i >= 4 ? br1 : br0, dst + i * 1024, b_voff[i & 3], kb + (MODE == 0 ? (i & 3) : i) * b_row8);
    } else {
#pragma unroll
      for (int i = I0; i < I1; ++i)
        ws_dma<NT>(MODE == 0 && i >= 4 ? br1 : br0, dst + i * 1024, b_voff[i & 3], kb + (MODE == 0 ? (i & 3) : i) * b_row8);
    }
  };
  auto issue_b_all = [&](int slot_b, int ks) __attribute__((always_inline)) {
    issue_b(std::integral_constant<int, 0>{}, std::integral_constant<int, WS_BQ>{}, slot_b, ks);
  };

  // ---- activation rows: instruction q of this wave fills tile rows 32 wave + 8 q + lane / 8
  // mode 0: the token of tile row 32 wave + lane (lanes < 32, clamped to the tile), loaded a step
  // before a_set needs it so that waiting for it does not drain the loads in flight
  auto tok_load = [&](const WsItem& d) __attribute__((always_inline)) {
    int t = 0;
    if (MODE == 0 && d.live) {
      const int r = min(wave * 32 + (lane_now() & 31), d.nrows - 1);
      t = d.sh ? d.row0 + r : row_token[d.row0 + r];
    }
    return t;
  };
  const bf16_t* a_base;
  int a_voff[WS_AQ], a_rot;
  auto a_set = [&](const WsItem& d, int tok_mine) __attribute__((always_inline)) {
    const int ln = lane_now();
    const int a_row = wave * 32 + (ln >> 3);  // tile row of this lane in instruction 0
    const int a_c0 = (ln & 7) ^ (ln >> 3);     // its source chunk, xor (q & 3) for instruction q
    a_base = MODE == 0 ? act_x : (d.sh ? h_shared_in : h_routed_in);
    a_rot = d.rot;
    const int row_bytes = (MODE == 0 ? D : (d.sh ? S : I)) * 2;
#pragma unroll
    for (int q = 0; q < WS_AQ; ++q) {
      const int c16 = (a_c0 ^ (q & 3)) << 4;
      int off = WS_OOB;
      if (MODE == 0) {
        const int tok = __shfl(tok_mine, q * 8 + (ln >> 3));
        if (d.live && a_row < d.nrows - q * 8) off = tok * row_bytes + c16;
      } else {
        if (d.live && a_row < d.nrows - q * 8) off = (d.row0 + a_row + q * 8) * row_bytes + c16;
      }
      a_voff[q] = off;
    }
  };
  auto issue_a = [&](int stage, int ks) __attribute__((always_inline)) {
    const int kb = kbytes(ks, a_rot);
    const __amdgpu_buffer_rsrc_t r = ws_rsrc(a_base, WS_RANGE);
    char* dst = lds + stage * WS_A_STAGE + wave * WS_AQ * 1024;
#pragma unroll
    for (int q = 0; q < WS_AQ; ++q) ws_dma<false>(r, dst + q * 1024, a_voff[q], kb);
  };

  // ---- multiply one step: acc[m][s] += A(rows 32 m ..) W(wave rows 32 s ..)^T over 64 k
  f32x16 acc[WS_NM][2];
  // fragment k-chunk kk * 2 + lh of row l32 (+ 32 per row group): one per-lane offset per kk
  int foff[WS_BK / 16];
#pragma unroll
  for (int kk = 0; kk < WS_BK / 16; ++kk) foff[kk] = ws_pos(l32, kk * 2 + lh);
  // Fragments of k-step kk + 1 are read while the MFMAs of kk run (two register sets); the
  // scheduling groups spread those reads between the MFMAs.
  // issue(kk) runs after the MFMAs of k-step kk: the step's loads go out between its MFMAs
  // instead of in one burst before them.
  auto compute = [&](auto nm, int stage, int slot_b, auto&& issue) __attribute__((always_inline)) {
    constexpr int NM = decltype(nm)::value;
    constexpr int KK = WS_BK / 16;
    const char* As = lds + stage * WS_A_STAGE;
    const char* Bs = wslab + slot_b * WS_SLAB;
    i32x4 fa[2][NM], fb[2][2];
    auto load = [&](int kk, int buf) __attribute__((always_inline)) {
      fb[buf][0] = *reinterpret_cast<const i32x4*>(Bs + foff[kk]);
      fb[buf][1] = *reinterpret_cast<const i32x4*>(Bs + 32 * 128 + foff[kk]);
#pragma unroll
      for (int m = 0; m < NM; ++m) fa[buf][m] = *reinterpret_cast<const i32x4*>(As + m * 32 * 128 + foff[kk]);
    };
    load(0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NM + 2, 0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cb = kk & 1;
      if (kk + 1 < KK) load(kk + 1, cb ^ 1);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        acc[m][0] = mfma32w(fa[cb][m], fb[cb][0], acc[m][0]);
        acc[m][1] = mfma32w(fa[cb][m], fb[cb][1], acc[m][1]);
      }
      issue(kk);
      if (kk + 1 < KK) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NM, 0);
      }
    }
  };
  // accumulator element q of lane: row 32 m + 8 (q / 4) + 4 lh + q % 4, weight row 32 s + l32 of the
  // wave. Stores go through a buffer resource spanning the item's rows, so rows past the tile's end
  // fall outside it and are dropped, and each store needs one offset register.
  auto epilogue = [&](const WsItem& d) __attribute__((always_inline)) {
    const int ld = MODE == 0 ? (d.sh ? S : I) : D;
    const __amdgpu_buffer_rsrc_t o = ws_rsrc((d.sh ? out_shared : out_routed) + (size_t)d.row0 * ld, d.nrows * ld * 2);
    const int ln = lane_now();
    const int vbase = ((ln >> 5) * 4 * ld + d.nt * HN + wave * (MODE == 0 ? 32 : 64) + (ln & 31)) * 2;
    const int row_bytes = ld * 2;
#pragma unroll
    for (int m = 0; m < WS_NM; ++m) {
      if (m * 32 >= d.nrows) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int voff = vbase + (m * 32 + (q >> 2) * 8 + (q & 3)) * row_bytes;
        if (MODE == 0) {
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(silu_mul(acc[m][0][q], acc[m][1][q])), o, voff, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(acc[m][0][q]), o, voff, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(acc[m][1][q]), o, voff + 64, 0, 0);
        }
      }
    }
  };

  // Step j of a group (j = 0..3, step n = 4 g + j of the item, its slab in slot sb): multiply
  // stage j with slab n, request stage n + 3 (into stage (j + 3) % 4, at a_ks of the activation
  // cursor's item) and slab n + 2 (into slot (sb + 2) % 3, at b_ks of the weight cursor's item).
  // Only the item's live 32-row groups (nm of them) are multiplied; the loads do not depend on nm.
  int sb = 0;  // slot of slab n
  auto step = [&](auto nm, int j, int a_ks, int b_ks) __attribute__((always_inline)) {
    wait_vmcnt<2 * WS_AQ + WS_BQ>();  // loads after slab n: stage n + 1, slab n + 1, stage n + 2
    wait_lgkm0();
    barrier_only();
    const int sbn = sb == 0 ? 2 : sb - 1;
    compute(nm, j, sb, [&](int kk) __attribute__((always_inline)) {
      using std::integral_constant;
      if (kk == 0) issue_b(integral_constant<int, 0>{}, integral_constant<int, 3>{}, sbn, b_ks);
      if (kk == 1) issue_b(integral_constant<int, 3>{}, integral_constant<int, 6>{}, sbn, b_ks);
      if (kk == 2) issue_b(integral_constant<int, 6>{}, integral_constant<int, WS_BQ>{}, sbn, b_ks);
      if (kk == 3) issue_a((j + 3) & 3, a_ks);
    });
    sb = sb == 2 ? 0 : sb + 1;
  };
  // One item's steps: the non-final groups (both cursors stay inside the item), then the final
  // group, in which the activation cursor moves to the next item after the first step and the
  // weight cursor after the second.
  auto run_item = [&](auto nm, const WsItem& next) __attribute__((always_inline)) {
    for (int g = 0; g < nk / 4 - 1; ++g) {
      const int k0 = 4 * g;
      step(nm, 0, k0 + 3, k0 + 2);
      step(nm, 1, k0 + 4, k0 + 3);
      step(nm, 2, k0 + 5, k0 + 4);
      step(nm, 3, k0 + 6, k0 + 5);
    }
    const int tok_next = tok_load(next);
    step(nm, 0, nk - 1, nk - 2);
    a_set(next, tok_next);
    step(nm, 1, 0, nk - 1);
    b_set(next);
    step(nm, 2, 1, 0);
    step(nm, 3, 2, 1);
  };

  // prologue, in the issue order of the steps before step 0 (weights, then activations): stage 0; slab 0,
  // stage 1; slab 1, stage 2
  WsItem cur = item_of(0);
  b_set(cur);
  a_set(cur, tok_load(cur));
  wait_vmcnt<0>();
  issue_a(0, 0);
  issue_b_all(0, 0);
  issue_a(1, 1);
  issue_b_all(1, 1);
  issue_a(2, 2);

  for (int i = 0; i < mine; ++i) {
#pragma unroll
    for (int m = 0; m < WS_NM; ++m)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[m][t][q] = 0.f;
    const WsItem next = item_of(i + 1);
    // a ragged tile multiplies only its live row groups (one code path per count, so the step
    // loop itself has no branches)
    const int nm = __builtin_amdgcn_readfirstlane(min(WS_NM, (cur.nrows + 31) >> 5));
    if (nm >= 4)
      run_item(std::integral_constant<int, 4>{}, next);
    else if (nm == 3)
      run_item(std::integral_constant<int, 3>{}, next);
    else if (nm == 2)
      run_item(std::integral_constant<int, 2>{}, next);
    else
      run_item(std::integral_constant<int, 1>{}, next);
    epilogue(cur);
    cur = next;
  }
  wait_vmcnt<0>();  // no LDS write may still be in flight when the block ends
}

bool wstream_ok(const Dims& d) {
  const int lds_max = device_lds_limit();
  const int64_t lim = WS_RANGE - (1 << 20);
  return d.dtype == 1 && WS_LDS <= (size_t)lds_max && d.D % 256 == 0 && d.I % 256 == 0 && d.S == d.I &&
         d.T * d.D * 2 < lim && d.R * d.I * 2 < lim && d.T * d.S * 2 < lim;
}

template <bool NT>
static hipError_t launch_wstream_nt(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s) {
  const void* k0 = (const void*)gemm_wstream_bf16<0, NT>;
  const void* k1 = (const void*)gemm_wstream_bf16<1, NT>;
  hipError_t attr = allow_dynamic_lds(k0, WS_LDS);
  if (attr == hipSuccess) attr = allow_dynamic_lds(k1, WS_LDS);
  if (attr != hipSuccess) return attr;  // never launch with more LDS than the kernel may take
  const int g0 = persistent_grid(k0, 64 * WS_WAVES, WS_LDS) & ~7;
  const int g1 = persistent_grid(k1, 64 * WS_WAVES, WS_LDS) & ~7;
  MOE_LAUNCH((gemm_wstream_bf16<0, NT>), dim3(g0), dim3(64 * WS_WAVES), WS_LDS, s, (const bf16_t*)a.x, nullptr,
             nullptr, a.row_token, a.offsets, a.tiles_wide, a.meta, (const bf16_t*)w.w1, (const bf16_t*)w.w3,
             (const bf16_t*)w.ws1, (const bf16_t*)w.ws3, (bf16_t*)a.h_routed, (bf16_t*)a.h_shared, (int)d.T, d.D, d.I,
             d.S, d.E);
  MOE_LAUNCH((gemm_wstream_bf16<1, NT>), dim3(g1), dim3(64 * WS_WAVES), WS_LDS, s, nullptr, (const bf16_t*)a.h_routed,
             (const bf16_t*)a.h_shared, a.row_token, a.offsets, a.tiles_wide, a.meta, (const bf16_t*)w.w2, nullptr,
             (const bf16_t*)w.ws2, nullptr, (bf16_t*)a.o_routed, (bf16_t*)a.o_shared, (int)d.T, d.D, d.I, d.S, d.E);
  return hipGetLastError();
}

hipError_t launch_wstream_bf16(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s) {
  // nontemporal weight loads while the routed experts average fewer rows than one M-tile
  if (d.R < (int64_t)WS_BM * d.E) return launch_wstream_nt<true>(d, w, a, s);
  return launch_wstream_nt<false>(d, w, a, s);
}

}  // namespace moe

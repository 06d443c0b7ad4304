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
// slab n + 1 and stage n + 2 in flight (activations first measured 1-2% slower). The step sequence
// runs on across the block's items without draining: an item's last steps request the next item's
// first stages. A ragged tile multiplies only its live 32-row groups.
//
// Tile kinds. The down projection runs on the 128-row tile list (kTk128; a dense layer of 1024
// tokens or more on the 256-row list with steps over all 256 rows, kTk256: the same weight slabs,
// two 32 KB activation stages issued one step ahead and first in their step, 256 accumulators per
// wave). Gate/up runs on the 256-row tile list with each tile as one or two 128-row halves
// (kTkPair): a tile of an expert with more than 128 rows alternates half-steps between its halves,
// both multiplying the same weight slab, so each weight byte is loaded once per 256 rows while the
// activation ring keeps its four 16 KB stages; a tile of at most 128 rows runs as kTk128 does.
// The per-expert tile height thus follows the expert's row count.
//
// Items to blocks. Each XCD's blocks take a contiguous range of the item list. Gate/up launches of
// enough tiles split it into runs of 16 blocks with equal shares of measured cost, a run's blocks
// taking its items in lockstep rounds of 16 (see the kernel); the others deal items by count.
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
constexpr int WS_BK = 64;                                            // k per step
constexpr int WS_NB = 3;                                             // weight slabs per wave
constexpr int WS_SLAB = WS_WROWS * WS_BK * 2;                        // 8 KB
constexpr int WS_BQ = WS_WROWS / 8;                                  // weight loads per wave and step
// Tile kinds: the 128-row tile list; the 256-row tile list with a step over all 256 rows; the
// 256-row tile list with each tile run as one or two 128-row halves that share the weight slabs.
constexpr int kTk128 = 0, kTk256 = 1, kTkPair = 2;
// per tile kind: rows of an activation stage, stages (4 of 16 KB, or 2 of 32 KB), loads per wave
// and step, 32-row groups, halves; the LDS holds the stages and then the slabs
template <int TK>
struct WsDims {
  static constexpr int ROWS = TK == kTk256 ? 256 : 128;
  static constexpr int NA = TK == kTk256 ? 2 : 4;
  static constexpr int A_STAGE = ROWS * WS_BK * 2;
  static constexpr int AQ = ROWS / 8 / WS_WAVES;
  static constexpr int NM = ROWS / 32;
  static constexpr int NH = TK == kTkPair ? 2 : 1;
  static constexpr int B0 = NA * A_STAGE;
  static constexpr size_t LDS = (size_t)B0 + (size_t)WS_WAVES * WS_NB * WS_SLAB;  // 160 KB
};
static_assert(WsDims<kTk128>::LDS == WsDims<kTk256>::LDS, "both stage heights fill the LDS alike");
constexpr size_t WS_LDS = WsDims<kTk128>::LDS;

typedef __bf16 bf16x8w_t __attribute__((ext_vector_type(8)));

MOE_DEV f32x16 mfma32w(i32x4 a, i32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8w_t, a), __builtin_bit_cast(bf16x8w_t, b), c,
                                                 0, 0, 0);
}

// NT: every weight load nontemporal (else only the tiles of single-M-tile experts). TK: the tile
// kind (kTk128, kTk256 or kTkPair, above).
template <int MODE, bool NT, int TK>
__global__ __launch_bounds__(64 * WS_WAVES) void gemm_wstream_bf16(
    const bf16_t* __restrict__ act_x, const bf16_t* __restrict__ h_routed_in, const bf16_t* __restrict__ h_shared_in,
    const int32_t* __restrict__ row_token, const int32_t* __restrict__ offsets, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ meta, const bf16_t* __restrict__ wa, const bf16_t* __restrict__ wb,
    const bf16_t* __restrict__ wsa, const bf16_t* __restrict__ wsb, bf16_t* __restrict__ out_routed,
    bf16_t* __restrict__ out_shared, int T, int D, int I, int S, int E) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  using W = WsDims<TK>;
  constexpr int WS_NA = W::NA, WS_A_STAGE = W::A_STAGE, WS_AQ = W::AQ, WS_NM = W::NM, WS_NH = W::NH, WS_B0 = W::B0;
  constexpr int LIST = TK == kTk128 ? kWideBM : kWideBM2;  // the tile list's rows per tile
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, lh = lane >> 5;
  constexpr int HN = MODE == 0 ? 128 : 256;  // output columns per item
  const int per_r = MODE == 0 ? I / HN : D / HN;
  const int per_s = MODE == 0 ? S / HN : D / HN;
  const int nr = meta[LIST == kWideBM ? 2 : 5];
  const int items = nr * per_r + (meta[LIST == kWideBM ? 3 : 6] - nr) * per_s;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
  // Gate/up (paired tiles): the blocks form runs of 16 (two per XCD), each run a contiguous range of
  // whole tiles holding an equal share of the launch's work. A tile's cost is its column items
  // times an item's measured time by kind (fitted to the blocks' end times at 4096 tokens, uniform
  // and skewed routing): a tile of at most 64 rows 12, of at most 128 rows 15, a paired tile (two
  // half-steps per k-step) 20, a tile of a routed expert with more than one (its weight tiles are
  // read by several blocks at once, mostly from L2) 17, a shared-expert tile 20. A run's 16 blocks
  // take its items in rounds of 16 consecutive ones (one tile's column items when a tile has 16), so
  // the items that run together are the ones the plain order runs together; a block's place in the
  // round moves by one each round, so no block always takes the same M-tile of an expert. Dealt by
  // count instead, the blocks that drew more paired tiles finished up to a quarter of the launch
  // after the rest.
  // Otherwise: this block's items are xcd * chunk + slot + i * per_xcd for i < mine (an XCD's
  // blocks share a range); gate/up ranges start at a multiple of per_r items (one tile's column
  // items), so the blocks that take a round's consecutive items share its activation rows.
  const int ntiles = meta[LIST == kWideBM ? 3 : 6];
  // (only with at least four tiles per run: a launch of few tiles would otherwise sit on few blocks)
  const bool runs = MODE == 0 && TK == kTkPair && per_xcd % kRunBlocks == 0 &&
                    ntiles >= 4 * ((int)gridDim.x / kRunBlocks);
  const int pos = slot % kRunBlocks;
  int run_lo = 0, run_hi = 0, chunk = 0, mine = 0;
  if (runs) {
    constexpr int kCostSmall = 12, kCostSingle = 15, kCostPaired = 20, kCostMulti = 17, kCostShared = 20;
    auto tile_cost = [&](int t) __attribute__((always_inline)) {
      if (t >= nr) return kCostShared * per_s;
      const Tile tl = tiles[t];
      const int c = offsets[tl.expert + 1] - offsets[tl.expert] > LIST ? kCostMulti
                    : tl.nrows > 128                                   ? kCostPaired
                    : tl.nrows > 64                                    ? kCostSingle
                                                                       : kCostSmall;
      return c * per_r;
    };
    auto tile_item = [&](int t) __attribute__((always_inline)) {
      return t < nr ? t * per_r : nr * per_r + (t - nr) * per_s;
    };
    const int run = xcd * (per_xcd / kRunBlocks) + slot / kRunBlocks;
    // the LDS is free until the prologue's loads
    if (ws_run_bounds(ntiles, items, run, (int)gridDim.x / kRunBlocks, tile_cost, tile_item,
                      reinterpret_cast<int*>(lds), run_lo, run_hi))
      mine = ws_run_count(run_lo, run_hi, pos);
  } else {
    chunk = MODE == 0 ? (((items + 7) >> 3) + per_r - 1) / per_r * per_r : (items + 7) >> 3;
    const int lim = min(chunk, items - xcd * chunk);
    mine = slot < lim ? (lim - slot + per_xcd - 1) / per_xcd : 0;
  }
  if (mine == 0) return;
  // the list index of this block's i-th item (i < mine)
  auto item_index = [&](int i) __attribute__((always_inline)) {
    return runs ? ws_run_item(run_lo, pos, i) : xcd * chunk + slot + i * per_xcd;
  };
  const int nk = (MODE == 0 ? D : I) / WS_BK;  // steps per item (the shared expert has S == I)

  auto item_of = [&](int i) __attribute__((always_inline)) {
    WsItem d;
    d.live = i < mine;
    d.row0 = 0, d.nrows = 0, d.nt = 0, d.expert = 0, d.rot = 0, d.sh = false, d.solo = false;
    if (d.live) {
      const WideItem it = wide_item<LIST>(item_index(i), tiles, nr, offsets, T, E, per_r, per_s);
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

  // ---- activation rows: instruction q of this wave fills stage rows RW wave + 8 q + lane / 8 (RW =
  // rows of a stage / 4); half hh (kTkPair) is tile rows 128 hh .. of the tile. Mode 0: the token of
  // stage row RW wave + lane (lanes < RW; kTkPair: lanes 32 .. 63 hold half 1's), clamped to the
  // tile, loaded a step before a_set needs it so that waiting for it does not drain the loads in flight
  constexpr int RW = W::ROWS / WS_WAVES;
  auto tok_load = [&](const WsItem& d) __attribute__((always_inline)) {
    int t = 0;
    if (MODE == 0 && d.live) {
      const int ln = lane_now();
      const int r = min(TK == kTkPair ? (ln >> 5) * 128 + wave * 32 + (ln & 31) : wave * RW + (ln & (RW - 1)),
                        d.nrows - 1);
      t = d.sh ? d.row0 + r : row_token[d.row0 + r];
    }
    return t;
  };
  const bf16_t* a_base;
  int a_voff[WS_NH][WS_AQ], a_rot;
  auto a_set = [&](const WsItem& d, int tok_mine) __attribute__((always_inline)) {
    const int ln = lane_now();
    const int a_c0 = (ln & 7) ^ (ln >> 3);  // the source chunk of instruction 0, xor (q & 3) for instruction q
    a_base = MODE == 0 ? act_x : (d.sh ? h_shared_in : h_routed_in);
    a_rot = d.rot;
    const int row_bytes = (MODE == 0 ? D : (d.sh ? S : I)) * 2;
#pragma unroll
    for (int hh = 0; hh < WS_NH; ++hh) {
      const int a_row = hh * 128 + wave * RW + (ln >> 3);  // tile row of this lane in instruction 0
#pragma unroll
      for (int q = 0; q < WS_AQ; ++q) {
        const int c16 = (a_c0 ^ (q & 3)) << 4;
        int off = WS_OOB;
        if (MODE == 0) {
          const int tok = __shfl(tok_mine, hh * 32 + q * 8 + (ln >> 3));
          if (d.live && a_row < d.nrows - q * 8) off = tok * row_bytes + c16;
        } else {
          if (d.live && a_row < d.nrows - q * 8) off = (d.row0 + a_row + q * 8) * row_bytes + c16;
        }
        a_voff[hh][q] = off;
      }
    }
  };
  // stage rows of half hh at step ks
  auto issue_a = [&](int stage, int ks, int hh) __attribute__((always_inline)) {
    const int kb = kbytes(ks, a_rot);
    const __amdgpu_buffer_rsrc_t r = ws_rsrc(a_base, WS_RANGE);
    char* dst = lds + stage * WS_A_STAGE + wave * WS_AQ * 1024;
    if (WS_NH == 1 || hh == 0) {
#pragma unroll
      for (int q = 0; q < WS_AQ; ++q) ws_dma<false>(r, dst + q * 1024, a_voff[0][q], kb);
    } else {
#pragma unroll
      for (int q = 0; q < WS_AQ; ++q) ws_dma<false>(r, dst + q * 1024, a_voff[WS_NH - 1][q], kb);
    }
  };

  // ---- multiply one step: acc[h][m][s] += A(rows 128 h + 32 m ..) W(wave rows 32 s ..)^T over 64 k
  f32x16 acc[WS_NH][WS_NM][2];
  // fragment k-chunk kk * 2 + lh of row l32 (+ 32 per row group): one per-lane offset per kk
  int foff[WS_BK / 16];
#pragma unroll
  for (int kk = 0; kk < WS_BK / 16; ++kk) foff[kk] = ws_pos(l32, kk * 2 + lh);
  // Fragments of k-step kk + 1 are read while the MFMAs of kk run (two register sets); the
  // scheduling groups spread those reads between the MFMAs.
  // issue(kk) runs after the MFMAs of k-step kk: the step's loads go out between its MFMAs
  // instead of in one burst before them.
  auto compute = [&](auto nm, auto hc, int stage, int slot_b, auto&& issue) __attribute__((always_inline)) {
    constexpr int NM = decltype(nm)::value;
    constexpr int H = decltype(hc)::value;
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
        acc[H][m][0] = mfma32w(fa[cb][m], fb[cb][0], acc[H][m][0]);
        acc[H][m][1] = mfma32w(fa[cb][m], fb[cb][1], acc[H][m][1]);
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
  // accumulator element q of lane: row 128 h + 32 m + 8 (q / 4) + 4 lh + q % 4, weight row 32 s + l32
  // of the wave. Stores go through a buffer resource spanning the item's rows, so rows past the
  // tile's end fall outside it and are dropped, and each store needs one offset register.
  auto epilogue = [&](const WsItem& d) __attribute__((always_inline)) {
    const int ld = MODE == 0 ? (d.sh ? S : I) : D;
    const __amdgpu_buffer_rsrc_t o = ws_rsrc((d.sh ? out_shared : out_routed) + (size_t)d.row0 * ld, d.nrows * ld * 2);
    const int ln = lane_now();
    const int vbase = ((ln >> 5) * 4 * ld + d.nt * HN + wave * (MODE == 0 ? 32 : 64) + (ln & 31)) * 2;
    const int row_bytes = ld * 2;
#pragma unroll
    for (int h = 0; h < WS_NH; ++h)
#pragma unroll
      for (int m = 0; m < WS_NM; ++m) {
        if (h * 128 + m * 32 >= d.nrows) continue;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int voff = vbase + (h * 128 + m * 32 + (q >> 2) * 8 + (q & 3)) * row_bytes;
          if (MODE == 0) {
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(silu_mul(acc[h][m][0][q], acc[h][m][1][q])), o, voff, 0,
                                                  0);
          } else {
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(acc[h][m][0][q]), o, voff, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(acc[h][m][1][q]), o, voff + 64, 0, 0);
          }
        }
      }
  };

  // Step j of a group (j = 0..3, step n = 4 g + j of the block's step sequence): multiply
  // activation stage n with the slab in slot sb, request loads of the slab two k-steps ahead (at
  // b_ks of the weight cursor's item, into slot (sb + 2) % 3) and the activation stage NA - 1 steps
  // ahead (half ah at k-step ak of the activation cursor's item).
  //   kTk128, kTkPair: stage n + 3 into stage (j + 3) % 4, issued after the step's weight loads;
  //   kTk256: stage n + 1 into stage (j + 1) % 2, issued before them (needed a step later).
  // kTkPair runs a tile of more than 128 rows as half-steps (half 0, then half 1 of each k-step,
  // both on that k-step's slab), each issuing half of a slab's loads: 8 loads where a step issues
  // 12. The wait leaves at most 16 younger loads in flight, which holds under either pattern and
  // wherever one follows the other. Only the live 32-row groups (nm of them) are multiplied; the
  // loads do not depend on nm.
  using std::integral_constant;
  using H0 = integral_constant<int, 0>;
  using H1 = integral_constant<int, 1>;
  int sb = 0;  // slot of the slab in use
  // a whole k-step (every tile of kTk128 and kTk256, the tiles of at most 128 rows of kTkPair)
  auto step = [&](auto nm, int j, int ak, int ah, int b_ks) __attribute__((always_inline)) {
    if constexpr (TK != kTk256)
      wait_vmcnt<2 * WS_AQ + WS_BQ>();  // loads after slab n: stage n + 1, slab n + 1, stage n + 2
    else
      wait_vmcnt<WS_BQ>();  // loads after stage n and slab n: slab n + 1
    wait_lgkm0();
    barrier_only();
    const int sbn = sb == 0 ? 2 : sb - 1;
    compute(nm, H0{}, j % WS_NA, sb, [&](int kk) __attribute__((always_inline)) {
      if constexpr (TK != kTk256) {
        if (kk == 0) issue_b(integral_constant<int, 0>{}, integral_constant<int, 3>{}, sbn, b_ks);
        if (kk == 1) issue_b(integral_constant<int, 3>{}, integral_constant<int, 6>{}, sbn, b_ks);
        if (kk == 2) issue_b(integral_constant<int, 6>{}, integral_constant<int, WS_BQ>{}, sbn, b_ks);
        if (kk == 3) issue_a((j + 3) & 3, ak, ah);
      } else {
        if (kk == 0) issue_a((j + 1) & 1, ak, 0);
        if (kk == 1) issue_b(integral_constant<int, 0>{}, integral_constant<int, 3>{}, sbn, b_ks);
        if (kk == 2) issue_b(integral_constant<int, 3>{}, integral_constant<int, 6>{}, sbn, b_ks);
        if (kk == 3) issue_b(integral_constant<int, 6>{}, integral_constant<int, WS_BQ>{}, sbn, b_ks);
      }
    });
    sb = sb == 2 ? 0 : sb + 1;
  };
  // a half-step of kTkPair: half H of the k-step, slab loads 4 H .. 4 H + 3 of step b_ks; the slot
  // moves on after half 1
  auto half_step = [&](auto nm, auto hc, int j, int ak, int ah, int b_ks) __attribute__((always_inline)) {
    constexpr int H = decltype(hc)::value;
    wait_vmcnt<2 * WS_AQ + WS_BQ>();
    wait_lgkm0();
    barrier_only();
    const int sbn = sb == 0 ? 2 : sb - 1;
    compute(nm, hc, j, sb, [&](int kk) __attribute__((always_inline)) {
      if (kk == 0) issue_b(integral_constant<int, 4 * H>{}, integral_constant<int, 4 * H + 2>{}, sbn, b_ks);
      if (kk == 1) issue_b(integral_constant<int, 4 * H + 2>{}, integral_constant<int, 4 * H + 4>{}, sbn, b_ks);
      if (kk == 3) issue_a((j + 3) & 3, ak, ah);
    });
    if (H == 1) sb = sb == 2 ? 0 : sb + 1;
  };
  auto paired = [&](const WsItem& d) __attribute__((always_inline)) {
    return TK == kTkPair && d.live && d.nrows > 128;
  };
  // (half, k-step) of step s of an item
  auto hk = [](bool pair, int s, int& h, int& k) __attribute__((always_inline)) {
    h = pair ? (s & 1) : 0;
    k = pair ? (s >> 1) : s;
  };
  // One item's steps: the non-final groups (both cursors stay inside the item), then the final
  // group, in which each cursor moves on to the next item once it passes the item's last step.
  auto run_item = [&](auto nm, const WsItem& next) __attribute__((always_inline)) {
    constexpr int LA = WS_NA - 1;  // steps the activation cursor runs ahead
    for (int g = 0; g < nk / 4 - 1; ++g) {
      const int k0 = 4 * g;
      step(nm, 0, k0 + LA, 0, k0 + 2);
      step(nm, 1, k0 + LA + 1, 0, k0 + 3);
      step(nm, 2, k0 + LA + 2, 0, k0 + 4);
      step(nm, 3, k0 + LA + 3, 0, k0 + 5);
    }
    if constexpr (TK != kTk256) {
      int h0, k0n, h1, k1n, h2, k2n;  // the next item's first three steps
      const bool np = paired(next);
      hk(np, 0, h0, k0n);
      hk(np, 1, h1, k1n);
      hk(np, 2, h2, k2n);
      const int tok_next = tok_load(next);
      step(nm, 0, nk - 1, 0, nk - 2);
      a_set(next, tok_next);
      step(nm, 1, k0n, h0, nk - 1);
      b_set(next);
      step(nm, 2, k1n, h1, 0);
      step(nm, 3, k2n, h2, 1);
    } else {
      step(nm, 0, nk - 3, 0, nk - 2);
      const int tok_next = tok_load(next);
      step(nm, 1, nk - 2, 0, nk - 1);
      b_set(next);
      step(nm, 2, nk - 1, 0, 0);
      a_set(next, tok_next);
      step(nm, 3, 0, 0, 1);
    }
  };
  // A kTkPair tile of more than 128 rows: half-steps 4 g + j = (half 0, k 2g), (half 1, k 2g),
  // (half 0, k 2g + 1), (half 1, k 2g + 1); half 0 is full, half 1 has nmb live row groups.
  auto run_pair = [&](auto nmb, const WsItem& next) __attribute__((always_inline)) {
    constexpr integral_constant<int, WS_NM> full{};
    for (int g = 0; g < nk / 2 - 1; ++g) {
      const int k0 = 2 * g;
      half_step(full, H0{}, 0, k0 + 1, 1, k0 + 2);
      half_step(nmb, H1{}, 1, k0 + 2, 0, k0 + 2);
      half_step(full, H0{}, 2, k0 + 2, 1, k0 + 3);
      half_step(nmb, H1{}, 3, k0 + 3, 0, k0 + 3);
    }
    int h0, k0n, h1, k1n, h2, k2n;
    const bool np = paired(next);
    hk(np, 0, h0, k0n);
    hk(np, 1, h1, k1n);
    hk(np, 2, h2, k2n);
    const int tok_next = tok_load(next);
    b_set(next);  // this item's last slab went out in the previous group
    half_step(full, H0{}, 0, nk - 1, 1, 0);
    a_set(next, tok_next);
    half_step(nmb, H1{}, 1, k0n, h0, 0);
    half_step(full, H0{}, 2, k1n, h1, 1);
    half_step(nmb, H1{}, 3, k2n, h2, 1);
  };

  // prologue, in the issue order of the steps before step 0: kTk128 and kTkPair: stage 0; slab 0,
  // stage 1; slab 1, stage 2 (weights, then activations); kTk256: slab 0; stage 0; slab 1
  WsItem cur = item_of(0);
  b_set(cur);
  a_set(cur, tok_load(cur));
  wait_vmcnt<0>();
  if constexpr (TK != kTk256) {
    int h, k;
    const bool cp = paired(cur);
    hk(cp, 0, h, k);
    issue_a(0, k, h);
    issue_b_all(0, 0);
    hk(cp, 1, h, k);
    issue_a(1, k, h);
    issue_b_all(1, 1);
    hk(cp, 2, h, k);
    issue_a(2, k, h);
  } else {
    issue_b_all(0, 0);
    issue_a(0, 0, 0);
    issue_b_all(1, 1);
  }

  for (int i = 0; i < mine; ++i) {
#pragma unroll
    for (int h = 0; h < WS_NH; ++h)
#pragma unroll
      for (int m = 0; m < WS_NM; ++m)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[h][m][t][q] = 0.f;
    const WsItem next = item_of(i + 1);
    // a ragged tile multiplies only its live row groups (one code path per count, so the step
    // loop itself has no branches)
    const int nm = __builtin_amdgcn_readfirstlane(min(WS_NM, (cur.nrows + 31) >> 5));
    if constexpr (TK == kTk256) {  // pairs of row groups (only the dense layer's last tile is ragged)
      if (nm >= 7)
        run_item(integral_constant<int, 8>{}, next);
      else if (nm >= 5)
        run_item(integral_constant<int, 6>{}, next);
      else if (nm >= 3)
        run_item(integral_constant<int, 4>{}, next);
      else
        run_item(integral_constant<int, 2>{}, next);
    } else {
      bool done = false;
      if constexpr (TK == kTkPair) {
        if (paired(cur)) {  // half 1's live row groups, rounded up to 2 or 4
          if (__builtin_amdgcn_readfirstlane(cur.nrows) > 128 + 64)
            run_pair(integral_constant<int, 4>{}, next);
          else
            run_pair(integral_constant<int, 2>{}, next);
          done = true;
        }
      }
      if (done) {
      } else if (nm >= 4) {
        run_item(integral_constant<int, 4>{}, next);
      } else if (nm == 3) {
        run_item(integral_constant<int, 3>{}, next);
      } else if (nm == 2) {
        run_item(integral_constant<int, 2>{}, next);
      } else {
        run_item(integral_constant<int, 1>{}, next);
      }
    }
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

// Gate/up on kTkPair tiles, down on TK1 tiles (kTk128; kTk256 for a large dense layer).
template <bool NT, int TK1>
static hipError_t launch_wstream_nt(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s) {
  const void* k0 = (const void*)gemm_wstream_bf16<0, NT, kTkPair>;
  const void* k1 = (const void*)gemm_wstream_bf16<1, NT, TK1>;
  hipError_t attr = allow_dynamic_lds(k0, WS_LDS);
  if (attr == hipSuccess) attr = allow_dynamic_lds(k1, WS_LDS);
  if (attr != hipSuccess) return attr;  // never launch with more LDS than the kernel may take
  const int g0 = persistent_grid(k0, 64 * WS_WAVES, WS_LDS) & ~7;
  const int g1 = persistent_grid(k1, 64 * WS_WAVES, WS_LDS) & ~7;
  MOE_LAUNCH((gemm_wstream_bf16<0, NT, kTkPair>), dim3(g0), dim3(64 * WS_WAVES), WS_LDS, s, (const bf16_t*)a.x,
             nullptr, nullptr, a.row_token, a.offsets, a.tiles_wide2, a.meta, (const bf16_t*)w.w1,
             (const bf16_t*)w.w3, (const bf16_t*)w.ws1, (const bf16_t*)w.ws3, (bf16_t*)a.h_routed,
             (bf16_t*)a.h_shared, (int)d.T, d.D, d.I, d.S, d.E);
  MOE_LAUNCH((gemm_wstream_bf16<1, NT, TK1>), dim3(g1), dim3(64 * WS_WAVES), WS_LDS, s, nullptr,
             (const bf16_t*)a.h_routed, (const bf16_t*)a.h_shared, a.row_token, a.offsets,
             TK1 == kTk128 ? a.tiles_wide : a.tiles_wide2, a.meta, (const bf16_t*)w.w2, nullptr,
             (const bf16_t*)w.ws2, nullptr, (bf16_t*)a.o_routed, (bf16_t*)a.o_shared, (int)d.T, d.D, d.I, d.S, d.E);
  return hipGetLastError();
}

// A dense layer of this many tokens or more runs its down projection on 256-row tiles: one weight
// matrix shared by every M-tile, all tiles full, activations that stay in L2, so the larger tile's
// third fewer bytes per flop through the load path win (4096 tokens, dim 7168, inter 18,432: down
// 1.09 -> 0.98 ms). With routed experts the 128-row down projection is the faster one.
constexpr int64_t kDenseTallRows = 1024;

hipError_t launch_wstream_bf16(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s) {
  if (d.E == 0 && d.T >= kDenseTallRows) return launch_wstream_nt<false, kTk256>(d, w, a, s);
  // nontemporal weight loads while the routed experts average fewer rows than one M-tile
  if (d.R < (int64_t)kWideBM * d.E) return launch_wstream_nt<true, kTk128>(d, w, a, s);
  return launch_wstream_nt<false, kTk128>(d, w, a, s);
}

}  // namespace moe

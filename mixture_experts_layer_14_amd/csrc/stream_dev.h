// Device code of the decode-sized bf16 expert GEMMs (16-row M-tiles, weights streamed through
// wave-private LDS slabs), shared by their kernels and the fused decode kernel. The SwiGLU expert of
// "DeepSeek-V3.2-Exp · Mixture of experts" (three dim x inter matrices per expert).
#pragma once
#include "kernels.h"

namespace moe {

constexpr int SK = 128;               // k per slab
constexpr int SLAB = 16 * SK * 2;     // bytes per slab (16 rows)

// 16 rows of 16 chunks: chunk c of row r at position c ^ r, so the 16 rows of one MFMA
// fragment read (one chunk each) hit 16 distinct positions.
MOE_DEV int slab_store_pos(int row, int ch) { return row * (SK * 2) + ((ch ^ row) << 4); }

// Per-wave streaming state for one weight matrix slice: 16 rows of `ldb` bytes, addressed through
// a buffer resource (base and byte range in scalar registers), so each lane needs a single 32-bit
// offset register and the row steps go into the scalar offset. Offsets at or past the range read
// as zero.
constexpr int kBufOob = 0x7fffffff;
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format

struct SlabStream {
  __amdgpu_buffer_rsrc_t rs;
  int ldb;
};

MOE_DEV SlabStream slab_stream(const bf16_t* rows, int ld) {
  return {__builtin_amdgcn_make_buffer_rsrc((void*)rows, (short)0, 16 * ld * 2, kBufFlags), ld * 2};
}

// Load slab k0 of one matrix, nontemporal: instruction i covers rows 4i + lane/16, chunk lane % 16.
// Lanes past K (a ragged last slab), and every lane when `live` is false, take an out-of-range
// offset and read zeros without touching memory; the instructions are issued either way, so
// every step issues the same loads (this keeps the compiler's load-count waits exact).
MOE_DEV void slab_load(i32x4 v[4], const SlabStream& st, int k0, int K, bool live, int lane) {
  const int q = lane >> 4, c = lane & 15;
  const int k = k0 + c * 8;
  const int off = (live && k < K) ? q * st.ldb + k * 2 : kBufOob;
  const int row4 = __builtin_amdgcn_readfirstlane(4 * st.ldb);  // uniform: keep it in a scalar register
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(st.rs, off, i * row4, 2));
}

MOE_DEV void slab_store(char* lds, const i32x4 v[4], int lane) {
  const int q = lane >> 4, c = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<i32x4*>(lds + slab_store_pos(4 * i + q, c)) = v[i];
}

MOE_DEV i32x4 slab_frag(const char* lds, int s, int lane) {
  const int r = lane & 15, q = lane >> 4;
  return *reinterpret_cast<const i32x4*>(lds + slab_store_pos(r, 4 * s + q));
}

// Sixteen zero bytes that A-fragment lanes past K read instead of masking after the load.
static __device__ __attribute__((aligned(16))) const bf16_t kZeroChunk[8] = {};

// A fragments of slab k0: lane (row r, q) takes k = k0 + 32 s + 8 q .. + 7 for step s; lanes
// past K read kZeroChunk. `arow` is always a readable row: rows past the tile's end read a real
// row whose products land only in output rows that are never stored (MFMA rows are
// independent), so they need no masking.
MOE_DEV void a_load(i32x4 a[4], const bf16_t* arow, int k0, int K, int lane) {
  typedef const __attribute__((address_space(1))) i32x4* global_i32x4;  // a global load, not a flat one
  const int q = lane >> 4;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int k = k0 + 32 * s + 8 * q;
    a[s] = *(global_i32x4)(k < K ? arow + k : kZeroChunk);
  }
}

// Multiply one landed slab (already in `lds`, NM matrices) with A fragments a: acc[m] += A W_m^T
// over k0 .. min(k0 + SK, K).
template <int NM>
MOE_DEV void slab_mma(f32x4 acc[NM], const i32x4 a[4], const char* lds, int k0, int K, int lane) {
  const int steps = min(4, (K - k0) >> 5);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < steps) {
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[m] = mfma_bf16_16x16x32(a[s], slab_frag(lds + m * SLAB, s, lane), acc[m]);
    }
  }
}

// How many of `workers` take `items` equal items round-robin: the fewest that still need only
// ceil(items / workers) rounds. Every worker's share is then that number of items or one less, so
// all of them finish together; with every worker busy, the few holding one item more than the
// rest would stream alone at the end, at a fraction of the bandwidth.
MOE_DEV int balanced_workers(int items, int workers) {
  if (items <= 0) return 0;
  const int rounds = (items + workers - 1) / workers;
  return (items + rounds - 1) / rounds;
}

// Both kernels run each wave through a flat sequence of steps (one slab of one item each) with
// two weight slabs in flight: step n multiplies the slab held in register set n % 2, after storing
// it to the wave's LDS slab and requesting slab n + 2 into the same registers. The request cursor
// runs on into the next item, so the weight stream does not drain at item boundaries.
//
// Vector-memory loads complete in issue order, so waiting for any load also waits for every
// older one. A fragments of step n + 1 (an L2 hit) are therefore requested before slab n + 2, into
// the second of two A register sets, and the step-n MFMAs wait only for loads issued before
// slab n + 1: two slabs really stay in flight.
MOE_DEV void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0): this wave's LDS traffic done
  __builtin_amdgcn_s_barrier();                                // loads in flight stay in flight
}

// mode 0: 8 waves per block split K; two slab sets, two A sets and the accumulators take ~146
// VGPRs, so one block (2 waves per SIMD) is resident per CU: 128 KB of weights in flight per CU.
// (4-wave blocks at 3 per CU, or 8-wave blocks held to 128 VGPRs with spills, measured slower.)
constexpr int G1_WAVES = 8;
// mode 1: 4 waves per block, each with its own items; ~100 registers, 4 blocks per CU (the rate
// did not change between 2 and 5 blocks per CU).
constexpr int G2_WAVES = 4;

// ---------------------------------------------------------------------------
// mode 0: gate/up + SwiGLU. Item = 16 rows x 16 h-columns; wave w of a block streams the w-th
// contiguous share of D (whole slabs) of every item of the block. At an item's end each wave parks
// its partial accumulators in its slab area and wave 0 reduces them in wave order.
// ---------------------------------------------------------------------------
struct G1Info {  // wave-uniform
  Tile tl;
  bool sh;
  int nt;
  SlabStream st[2];
};

MOE_DEV G1Info g1_info(int item, const Tile* tiles, int nr, int per_r, int per_s, const bf16_t* w1,
                       const bf16_t* w3, const bf16_t* ws1, const bf16_t* ws3, int D, int I, int E) {
  G1Info g;
  int ti;
  if (item < nr * per_r) {
    ti = item / per_r;
    g.nt = item % per_r;
  } else {
    ti = nr + (item - nr * per_r) / per_s;
    g.nt = (item - nr * per_r) % per_s;
  }
  g.tl = tiles[ti];
  g.sh = g.tl.expert == E;
  const size_t eoff = g.sh ? 0 : (size_t)g.tl.expert * I * D;
  g.st[0] = slab_stream((g.sh ? ws1 : w1 + eoff) + (size_t)g.nt * 16 * D, D);
  g.st[1] = slab_stream((g.sh ? ws3 : w3 + eoff) + (size_t)g.nt * 16 * D, D);
  return g;
}

// x row of this lane's tile row (rows past the tile's end read token 0)
MOE_DEV const bf16_t* g1_arow(const G1Info& g, const bf16_t* x, const int32_t* row_token, int D, int r) {
  int tok = 0;
  if (r < g.tl.nrows) tok = g.sh ? g.tl.row0 + r : row_token[g.tl.row0 + r];
  return x + (size_t)tok * D;
}

// The kernel body as block `bid` of `nblocks` (the items of a block: bid, bid + nblocks, ...); lds:
// G1_WAVES x 2 slabs.
MOE_DEV void gemm1_stream_run(int bid, int nblocks, char (*lds)[2 * SLAB], const bf16_t* __restrict__ x,
                              const int32_t* __restrict__ row_token, const Tile* __restrict__ tiles,
                              const int32_t* __restrict__ meta, const bf16_t* __restrict__ w1,
                              const bf16_t* __restrict__ w3, const bf16_t* __restrict__ ws1,
                              const bf16_t* __restrict__ ws3, bf16_t* __restrict__ h_routed,
                              bf16_t* __restrict__ h_shared, int D, int I, int S, int E) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int per_r = I / 16, per_s = S / 16;
  const int nr = meta[0];
  const int items = nr * per_r + (meta[1] - nr) * per_s;
  // contiguous k-range of this wave, in whole slabs (empty when D has fewer slabs than waves)
  const int nslab = (D + SK - 1) / SK;
  const int kb = (nslab * wave / G1_WAVES) * SK;
  const int ke = min(D, (nslab * (wave + 1) / G1_WAVES) * SK);
  // the items of block b: b, b + nblocks, ... over the blocks that take part
  nblocks = balanced_workers(items, nblocks);
  int item = bid;
  if (item >= nblocks) return;
  f32x4* red = reinterpret_cast<f32x4*>(lds[wave]);
  auto info_at = [&](int it) { return g1_info(it, tiles, nr, per_r, per_s, w1, w3, ws1, ws3, D, I, E); };

  // At an item's end: partials to LDS, wave 0 reduces in wave order, applies SwiGLU and stores.
  auto finish = [&](const G1Info& c, const f32x4 acc[2]) {
    red[lane] = acc[0];
    red[64 + lane] = acc[1];
    lds_barrier();
    if (wave == 0) {
      f32x4 g = acc[0], u = acc[1];
#pragma unroll
      for (int w = 1; w < G1_WAVES; ++w) {
        const f32x4* rw = reinterpret_cast<const f32x4*>(lds[w]);
        g += rw[lane];
        u += rw[64 + lane];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = q * 4 + i;
        if (row < c.tl.nrows) {
          bf16_t* dst = c.sh ? h_shared + (size_t)(c.tl.row0 + row) * S : h_routed + (size_t)(c.tl.row0 + row) * I;
          dst[c.nt * 16 + r] = f32_to_bf16(silu_mul(g[i], u[i]));
        }
      }
    }
    lds_barrier();
  };

  if (kb >= ke) {  // no slabs for this wave: take part in every item's reduction with zeros
    const f32x4 zero[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    for (; item < items; item += nblocks) finish(info_at(item), zero);
    return;
  }

  // request cursor (slab n + 2)
  int l_item = item, l_k0 = kb;
  G1Info l = info_at(l_item);
  auto request = [&](i32x4 v[2][4]) {  // past the block's last item: zeros, no traffic
    const bool live = l_item < items;
    slab_load(v[0], l.st[0], l_k0, ke, live, lane);
    slab_load(v[1], l.st[1], l_k0, ke, live, lane);
    if (!live) return;
    l_k0 += SK;
    if (l_k0 >= ke) {
      l_item += nblocks;
      l_k0 = kb;
      if (l_item < items) l = info_at(l_item);
    }
  };
  // A cursor (step n + 1)
  int p_item = item, p_k0 = kb;
  const bf16_t* p_arow = g1_arow(l, x, row_token, D, r);
  auto a_next = [&](i32x4 a[4]) {
    const bool live = p_item < items;
    a_load(a, p_arow, p_k0, live ? ke : 0, lane);
    if (!live) return;
    p_k0 += SK;
    if (p_k0 >= ke) {
      p_item += nblocks;
      p_k0 = kb;
      if (p_item < items) p_arow = g1_arow(info_at(p_item), x, row_token, D, r);
    }
  };
  i32x4 v0[2][4], v1[2][4], a0[4], a1[4];
  // same issue order as the steady state (A of a step goes out between the two slabs ahead)
  request(v0);
  a_next(a0);
  request(v1);
  // compute cursor (step n)
  G1Info c = info_at(item);
  int c_k0 = kb;
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  // One step on register sets v / a (A of the following step goes to an). Every step issues the
  // same loads, and the loop has a single exit after the second step of a trip: otherwise the
  // compiler merges a load-free or early-exit path into the loop head and waits there for every
  // load in flight. A step after the last item only issues (empty) loads.
  bool done = false;
  auto step = [&](i32x4 v[2][4], const i32x4 a[4], i32x4 an[4]) {
    slab_store(lds[wave], v[0], lane);
    slab_store(lds[wave] + SLAB, v[1], lane);
    a_next(an);
    request(v);
    if (done) return;
    slab_mma<2>(acc, a, lds[wave], c_k0, ke, lane);
    c_k0 += SK;
    if (c_k0 >= ke) {
      finish(c, acc);
      acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
      item += nblocks;
      done = item >= items;
      if (!done) c = info_at(item);
      c_k0 = kb;
    }
  };
  for (;;) {  // two steps per trip so the register sets alternate statically
    step(v0, a0, a1);
    step(v1, a1, a0);
    if (done) return;
  }
}


// ---------------------------------------------------------------------------
// mode 1: down projection. Each wave owns whole items of 16 rows x 16 output columns and walks
// its items as one continuous weight stream.
// ---------------------------------------------------------------------------
struct G2Info {  // wave-uniform
  Tile tl;
  bool sh;
  int nt, ks, K, ld, rot;  // K: the item's k length (one split's share), ld: the row stride
  SlabStream st;
};

// Physical k of logical k offset k0 of item g. Items start their k walk at different slabs: with
// every wave at the same offset of 4 KB-strided rows, concurrent requests bunch on a few HBM
// channels (measured: 6.4 TB/s in step, 6.7 TB/s staggered).
MOE_DEV int g2_k(const G2Info& g, int k0) {
  const int k = k0 + g.rot;
  return k >= g.K ? k - g.K : k;
}

// item -> (tile, 16-column group nt, k split ks): with ksplit > 1 each item covers the ks-th share
// of k, reading weights and h from that share's first column on (same row strides).
MOE_DEV G2Info g2_info(int item, const Tile* tiles, int per, int ksplit, const bf16_t* w2, const bf16_t* ws2, int D,
                       int I, int S, int E) {
  G2Info g;
  const int base = item / ksplit;
  g.ks = item - base * ksplit;
  const int ti = base / per;
  g.nt = base % per;
  g.tl = tiles[ti];
  g.sh = g.tl.expert == E;
  g.ld = g.sh ? S : I;
  g.K = g.ld / ksplit;
  g.st = slab_stream((g.sh ? ws2 : w2 + (size_t)g.tl.expert * D * I) + (size_t)g.nt * 16 * g.ld + (size_t)g.ks * g.K,
                     g.ld);
  g.rot = g.K % SK == 0 ? ((g.nt * 5 + g.tl.expert * 3) % (g.K / SK)) * SK : 0;
  return g;
}

// h row of this lane's tile row (rows past the tile's end read the tile's row 0), from the
// item's k share on
MOE_DEV const bf16_t* g2_arow(const G2Info& g, const bf16_t* h_routed, const bf16_t* h_shared, int r) {
  const bf16_t* A = g.sh ? h_shared : h_routed;
  return A + (size_t)(g.tl.row0 + (r < g.tl.nrows ? r : 0)) * g.ld + (size_t)g.ks * g.K;
}

// ksplit == 1: o = h W2^T in bf16. ksplit > 1 (shared-expert tiles only): split ks writes its fp32
// partial sum to part[ks][token][column]; dense_down_sum adds the splits in order.
// The kernel body on NW waves as block `bid` of `nblocks` (each wave its own items); lds: NW slabs.
template <int NW>
MOE_DEV void gemm2_stream_run(int bid, int nblocks, char (*lds)[SLAB], const bf16_t* __restrict__ h_routed,
                              const bf16_t* __restrict__ h_shared, const Tile* __restrict__ tiles,
                              const int32_t* __restrict__ meta, const bf16_t* __restrict__ w2,
                              const bf16_t* __restrict__ ws2, bf16_t* __restrict__ o_routed,
                              bf16_t* __restrict__ o_shared, float* __restrict__ part, int ksplit, int T, int D,
                              int I, int S, int E) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int per = D / 16;
  const int items = meta[1] * per * ksplit;
  // the items of wave w: w, w + stride, ... over the waves that take part
  const int stride = balanced_workers(items, nblocks * NW);
  int item = bid * NW + wave;
  if (item >= stride) return;
  auto info_at = [&](int it) { return g2_info(it, tiles, per, ksplit, w2, ws2, D, I, S, E); };

  int l_item = item, l_k0 = 0;
  G2Info l = info_at(l_item);
  auto request = [&](i32x4 v[4]) {
    const bool live = l_item < items;
    slab_load(v, l.st, g2_k(l, l_k0), l.K, live, lane);
    if (!live) return;
    l_k0 += SK;
    if (l_k0 >= l.K) {
      l_item += stride;
      l_k0 = 0;
      if (l_item < items) l = info_at(l_item);
    }
  };
  int p_item = item, p_k0 = 0;
  G2Info p = l;
  const bf16_t* p_arow = g2_arow(p, h_routed, h_shared, r);
  auto a_next = [&](i32x4 a[4]) {
    const bool live = p_item < items;
    a_load(a, p_arow, g2_k(p, p_k0), live ? p.K : 0, lane);
    if (!live) return;
    p_k0 += SK;
    if (p_k0 >= p.K) {
      p_item += stride;
      p_k0 = 0;
      if (p_item < items) {
        p = info_at(p_item);
        p_arow = g2_arow(p, h_routed, h_shared, r);
      }
    }
  };
  i32x4 v0[4], v1[4], a0[4], a1[4];
  // same issue order as the steady state (A of a step goes out between the two slabs ahead)
  request(v0);
  a_next(a0);
  request(v1);
  G2Info c = info_at(item);
  int c_k0 = 0;
  f32x4 acc[1] = {{0.f, 0.f, 0.f, 0.f}};
  bool done = false;  // same step and loop shape as mode 0
  auto step = [&](i32x4 v[4], const i32x4 a[4], i32x4 an[4]) {
    slab_store(lds[wave], v, lane);
    a_next(an);
    request(v);
    if (done) return;
    slab_mma<1>(acc, a, lds[wave], g2_k(c, c_k0), c.K, lane);
    c_k0 += SK;
    if (c_k0 >= c.K) {
      if (ksplit == 1) {
        bf16_t* O = c.sh ? o_shared : o_routed;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = q * 4 + i;
          if (row < c.tl.nrows) O[(size_t)(c.tl.row0 + row) * D + c.nt * 16 + r] = f32_to_bf16(acc[0][i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = q * 4 + i;
          if (row < c.tl.nrows) part[((size_t)c.ks * T + c.tl.row0 + row) * D + c.nt * 16 + r] = acc[0][i];
        }
      }
      acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      item += stride;
      done = item >= items;
      if (!done) c = info_at(item);
      c_k0 = 0;
    }
  };
  for (;;) {
    step(v0, a0, a1);
    step(v1, a1, a0);
    if (done) return;
  }
}

}  // namespace moe

// Decode-sized expert GEMMs in bf16 (M-tiles of at most 16 rows): the SwiGLU expert of
// "DeepSeek-V3.2-Exp · Mixture of experts" (three dim x inter matrices per expert) when each
// expert sees a handful of tokens and the block is bound by reading the touched experts'
// weights from HBM once.
//
//   mode 0 (gate/up): h[rows, 16 cols] = silu(A W1^T) * (A W3^T), A = gathered x rows
//   mode 1 (down):    O[rows, 16 cols] = h W2^T
//
// Weights stream through a wave-private LDS slab of 16 rows x 128 k: one wave instruction
// reads 4 rows x 256 contiguous bytes with nontemporal loads (the pattern HBM serves best),
// the slab is stored with 16-byte chunks XOR-swizzled by row and read back in MFMA B layout
// (lane: row = lane % 16, k-chunk 4 s + lane / 16 for 16x16x32 step s). The next slab's loads
// are in flight while the current one is multiplied. A fragments (x or h rows, a few KB,
// L2-resident) use the same k mapping.
//
// Mode 0 splits K = dim over the 8 waves of a 512-thread block and reduces the partial
// accumulators through LDS in wave order; mode 1 gives each wave a whole 16-column item.
#include "kernels.h"

namespace moe {

constexpr int SK = 128;               // k per slab
constexpr int SLAB = 16 * SK * 2;     // bytes per slab (16 rows)
constexpr int G1_WAVES = 8;           // mode 0: waves per block (K split)
constexpr int G2_WAVES = 4;           // mode 1: waves per block (independent items)

MOE_DEV i32x4 nt_ld16(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p)); }

// 16 rows of 16 chunks: chunk c of row r at position c ^ r, so the 16 rows of one MFMA
// fragment read (one chunk each) hit 16 distinct positions.
MOE_DEV int slab_store_pos(int row, int ch) { return row * (SK * 2) + ((ch ^ row) << 4); }

// Per-wave streaming state for one weight matrix slice: 16 rows starting at `w`, row stride `ld`.
struct SlabStream {
  const bf16_t* w;
  int ld;
};

// Load slab k0 of one matrix: instruction i covers rows 4i + lane/16, chunk lane % 16.
MOE_DEV void slab_load(i32x4 v[4], const SlabStream& st, int k0, int K, int lane) {
  const int q = lane >> 4, c = lane & 15;
  const int k = k0 + c * 8;
  const i32x4 zero = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = k < K ? nt_ld16(st.w + (size_t)(4 * i + q) * st.ld + k) : zero;
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

// A fragments of slab k0: lane (row r, q) takes k = k0 + 32 s + 8 q .. + 7 for step s.
MOE_DEV void a_load(i32x4 a[4], const bf16_t* arow, bool valid, int k0, int K, int lane) {
  const int q = lane >> 4;
  const i32x4 zero = {0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int k = k0 + 32 * s + 8 * q;
    a[s] = (valid && k < K) ? ld16(arow + k) : zero;
  }
}

// One wave's pass over k-range [kb, ke) (multiples of SK except a final ragged end):
// accumulates acc[m] += A * W_m^T for NM matrices.
template <int NM>
MOE_DEV void stream_range(f32x4 acc[NM], const SlabStream st[NM], const bf16_t* arow, bool avalid, int kb, int ke,
                          int K, char* lds /* NM slabs */, int lane) {
  if (kb >= ke) return;
  i32x4 v[NM][4], a[4], an[4];
#pragma unroll
  for (int m = 0; m < NM; ++m) slab_load(v[m], st[m], kb, ke, lane);
  a_load(a, arow, avalid, kb, ke, lane);
  for (int k0 = kb; k0 < ke; k0 += SK) {
#pragma unroll
    for (int m = 0; m < NM; ++m) slab_store(lds + m * SLAB, v[m], lane);
    const bool more = k0 + SK < ke;
    if (more) {
#pragma unroll
      for (int m = 0; m < NM; ++m) slab_load(v[m], st[m], k0 + SK, ke, lane);
      a_load(an, arow, avalid, k0 + SK, ke, lane);
    }
    const int steps = min(4, (ke - k0) >> 5);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < steps) {
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[m] = mfma_bf16_16x16x32(a[s], slab_frag(lds + m * SLAB, s, lane), acc[m]);
      }
    }
    if (more) {
#pragma unroll
      for (int s = 0; s < 4; ++s) a[s] = an[s];
    }
  }
  (void)K;
}

// ---------------------------------------------------------------------------
// mode 0: gate/up + SwiGLU. Block = 8 waves = one item (16 rows x 16 h-columns); wave w
// streams the w-th contiguous eighth of D (whole slabs). After the pass each wave's slab
// buffer holds its partial accumulators for the in-order reduction by wave 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64 * G1_WAVES, 4) void gemm1_stream_bf16(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ row_token, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ meta, const bf16_t* __restrict__ w1, const bf16_t* __restrict__ w3,
    const bf16_t* __restrict__ ws1, const bf16_t* __restrict__ ws3, bf16_t* __restrict__ h_routed,
    bf16_t* __restrict__ h_shared, int D, int I, int S, int E) {
  __shared__ __attribute__((aligned(16))) char lds[G1_WAVES][2 * SLAB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int per_r = I / 16, per_s = S / 16;
  const int nr = meta[0];
  const int items = nr * per_r + (meta[1] - nr) * per_s;
  // contiguous k-range of this wave, in whole slabs
  const int nslab = (D + SK - 1) / SK;
  const int kb = (nslab * wave / G1_WAVES) * SK;
  const int ke = min(D, (nslab * (wave + 1) / G1_WAVES) * SK);
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    int ti, nt;
    if (item < nr * per_r) {
      ti = item / per_r;
      nt = item % per_r;
    } else {
      ti = nr + (item - nr * per_r) / per_s;
      nt = (item - nr * per_r) % per_s;
    }
    const Tile tl = tiles[ti];
    const bool sh = tl.expert == E;
    const size_t eoff = sh ? 0 : (size_t)tl.expert * I * D;
    SlabStream st[2] = {{(sh ? ws1 : w1 + eoff) + (size_t)nt * 16 * D, D},
                        {(sh ? ws3 : w3 + eoff) + (size_t)nt * 16 * D, D}};
    const bool av = r < tl.nrows;
    int tok = 0;
    if (av) tok = sh ? tl.row0 + r : row_token[tl.row0 + r];
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    stream_range<2>(acc, st, x + (size_t)tok * D, av, kb, ke, D, lds[wave], lane);
    f32x4* red = reinterpret_cast<f32x4*>(lds[wave]);  // this wave is done with its slabs
    red[lane] = acc[0];
    red[64 + lane] = acc[1];
    __syncthreads();
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
        if (row < tl.nrows) {
          bf16_t* dst = sh ? h_shared + (size_t)(tl.row0 + row) * S : h_routed + (size_t)(tl.row0 + row) * I;
          dst[nt * 16 + r] = f32_to_bf16(silu_mul(g[i], u[i]));
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// mode 1: down projection. Each wave owns whole items of 16 rows x 16 output columns.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64 * G2_WAVES) void gemm2_stream_bf16(
    const bf16_t* __restrict__ h_routed, const bf16_t* __restrict__ h_shared, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ meta, const bf16_t* __restrict__ w2, const bf16_t* __restrict__ ws2,
    bf16_t* __restrict__ o_routed, bf16_t* __restrict__ o_shared, int D, int I, int S, int E) {
  __shared__ __attribute__((aligned(16))) char lds[G2_WAVES][SLAB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int per = D / 16;
  const int items = meta[1] * per;
  for (int item = blockIdx.x * G2_WAVES + wave; item < items; item += gridDim.x * G2_WAVES) {
    const int ti = item / per, nt = item % per;
    const Tile tl = tiles[ti];
    const bool sh = tl.expert == E;
    const int K = sh ? S : I;
    const bf16_t* A = sh ? h_shared + (size_t)tl.row0 * S : h_routed + (size_t)tl.row0 * I;
    SlabStream st[1] = {{(sh ? ws2 : w2 + (size_t)tl.expert * D * I) + (size_t)nt * 16 * K, K}};
    const bool av = r < tl.nrows;
    f32x4 acc[1] = {{0.f, 0.f, 0.f, 0.f}};
    stream_range<1>(acc, st, A + (size_t)(av ? r : 0) * K, av, 0, K, K, lds[wave], lane);
    bf16_t* O = sh ? o_shared : o_routed;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = q * 4 + i;
      if (row < tl.nrows) O[(size_t)(tl.row0 + row) * D + nt * 16 + r] = f32_to_bf16(acc[0][i]);
    }
  }
}

hipError_t launch_stream_bf16(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s) {
  const int g1 = persistent_grid((const void*)gemm1_stream_bf16, 64 * G1_WAVES);
  const int g2 = persistent_grid((const void*)gemm2_stream_bf16, 64 * G2_WAVES);
  MOE_LAUNCH(gemm1_stream_bf16, dim3(g1), dim3(64 * G1_WAVES), 0, s, (const bf16_t*)a.x, a.row_token, a.tiles_skinny,
             a.meta, (const bf16_t*)w.w1, (const bf16_t*)w.w3, (const bf16_t*)w.ws1, (const bf16_t*)w.ws3,
             (bf16_t*)a.h_routed, (bf16_t*)a.h_shared, d.D, d.I, d.S, d.E);
  MOE_LAUNCH(gemm2_stream_bf16, dim3(g2), dim3(64 * G2_WAVES), 0, s, (const bf16_t*)a.h_routed,
             (const bf16_t*)a.h_shared, a.tiles_skinny, a.meta, (const bf16_t*)w.w2, (const bf16_t*)w.ws2,
             (bf16_t*)a.o_routed, (bf16_t*)a.o_shared, d.D, d.I, d.S, d.E);
  return hipGetLastError();
}

}  // namespace moe

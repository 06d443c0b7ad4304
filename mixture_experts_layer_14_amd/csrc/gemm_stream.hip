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
// (lane: row = lane % 16, k-chunk 4 s + lane / 16 for 16x16x32 step s). Two slabs per wave are
// in flight while the current one is multiplied, across item boundaries. A fragments (x or h
// rows, a few KB, L2-resident) use the same k mapping.
//
// Mode 0 splits K = dim over the 8 waves of a 512-thread block and reduces the partial
// accumulators through LDS in wave order; mode 1 gives each wave whole 16-column items.
#include "stream_dev.h"

namespace moe {

__global__ __launch_bounds__(64 * G1_WAVES, 2) void gemm1_stream_bf16(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ row_token, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ meta, const bf16_t* __restrict__ w1, const bf16_t* __restrict__ w3,
    const bf16_t* __restrict__ ws1, const bf16_t* __restrict__ ws3, bf16_t* __restrict__ h_routed,
    bf16_t* __restrict__ h_shared, int D, int I, int S, int E) {
  __shared__ __attribute__((aligned(16))) char lds[G1_WAVES][2 * SLAB];
  gemm1_stream_run(blockIdx.x, gridDim.x, lds, x, row_token, tiles, meta, w1, w3, ws1, ws3, h_routed, h_shared, D, I,
                   S, E);
}

__global__ __launch_bounds__(64 * G2_WAVES) void gemm2_stream_bf16(
    const bf16_t* __restrict__ h_routed, const bf16_t* __restrict__ h_shared, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ meta, const bf16_t* __restrict__ w2, const bf16_t* __restrict__ ws2,
    bf16_t* __restrict__ o_routed, bf16_t* __restrict__ o_shared, float* __restrict__ part, int ksplit, int T, int D,
    int I, int S, int E) {
  __shared__ __attribute__((aligned(16))) char lds[G2_WAVES][SLAB];
  gemm2_stream_run<G2_WAVES>(blockIdx.x, gridDim.x, lds, h_routed, h_shared, tiles, meta, w2, ws2, o_routed, o_shared,
                             part, ksplit, T, D, I, S, E);
}

// out[t][c] = bf16( sum over ks ascending of part[ks][t][c] ), fp32 adds
__global__ __launch_bounds__(256) void dense_down_sum(const float* __restrict__ part, int ksplit, int64_t n,
                                                      bf16_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float v = part[i];
    for (int ks = 1; ks < ksplit; ++ks) v += part[(size_t)ks * n + i];
    out[i] = f32_to_bf16(v);
  }
}

int dense_down_split(const Dims& d) {
  // the dense feed-forward's down projection on the 16-row path has ceil(T/16) * D/16 items of
  // the full inter length; split k until there are about two items per SIMD (keeping the split a
  // divisor of inter / 128). At 16 tokens this gives 4 shares (1,792 items): 0.165 ms per dense
  // step against 0.168 ms with 9 shares (4,032 items) and 0.170 ms with 16.
  if (d.E != 0 || d.dtype != 1 || d.T <= 0 || d.T >= kDenseWideRows || d.S % SK || d.D < 16) return 1;
  const int64_t items = (d.T + 15) / 16 * (d.D / 16);
  int want = (int)std::min<int64_t>(16, (2048 + items - 1) / items);
  while (want > 1 && (d.S / SK) % want) --want;
  return want;
}

hipError_t launch_stream_bf16(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s) {
  const int g1 = persistent_grid((const void*)gemm1_stream_bf16, 64 * G1_WAVES);
  const int g2 = persistent_grid((const void*)gemm2_stream_bf16, 64 * G2_WAVES);
  MOE_LAUNCH(gemm1_stream_bf16, dim3(g1), dim3(64 * G1_WAVES), 0, s, (const bf16_t*)a.x, a.row_token, a.tiles_skinny,
             a.meta, (const bf16_t*)w.w1, (const bf16_t*)w.w3, (const bf16_t*)w.ws1, (const bf16_t*)w.ws3,
             (bf16_t*)a.h_routed, (bf16_t*)a.h_shared, d.D, d.I, d.S, d.E);
  const int split = dense_down_split(d);
  if (split > 1 && !a.part) return hipErrorInvalidValue;  // the caller sized no partial buffer
  MOE_LAUNCH(gemm2_stream_bf16, dim3(g2), dim3(64 * G2_WAVES), 0, s, (const bf16_t*)a.h_routed,
             (const bf16_t*)a.h_shared, a.tiles_skinny, a.meta, (const bf16_t*)w.w2, (const bf16_t*)w.ws2,
             (bf16_t*)a.o_routed, (bf16_t*)a.o_shared, a.part, split, (int)d.T, d.D, d.I, d.S, d.E);
  if (split > 1) {
    const int64_t n = d.T * d.D;
    MOE_LAUNCH(dense_down_sum, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 2048)), dim3(256), 0, s, a.part,
               split, n, (bf16_t*)a.o_shared);
  }
  return hipGetLastError();
}

}  // namespace moe

// Dispatch of the MoE block ("DeepSeek-V3.2-Exp · Mixture of experts", MoE.forward
// excerpt: bincount of the chosen experts, then for each expert the tokens that chose
// it, in token order). Deterministic: counts come from per-block bitmaps, positions
// from an exclusive scan plus a popcount rank; no atomic decides an output position.
//
// Three launches over blocks of 256 tokens:
//   count:   per block, an LDS bitmap bits[e][256 tokens] -> blk[b][e] = popcount
//   scan:    one workgroup: blk[b][e] -> base row of block b inside expert e,
//            counts, offsets, and the GEMM tile lists (M-tiles of 16, 128 and 256 rows)
//   scatter: rebuilds the bitmap; row = base + popcount of earlier tokens' bits
// Up to 256 tokens (one block) all three run in a single workgroup (dispatch_single).
#include "dispatch_dev.h"

namespace moe {

__global__ __launch_bounds__(TB) void dispatch_count(const int32_t* __restrict__ idx, int T, int K, int E,
                                                     int32_t* __restrict__ blk) {
  extern __shared__ unsigned long long bits[];
  build_bits(bits, idx, T, K, E, blockIdx.x);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < WORDS; ++w) c += __popcll(bits[e * WORDS + w]);
    blk[(size_t)blockIdx.x * E + e] = c;
  }
}

__global__ __launch_bounds__(256) void dispatch_scan(int32_t* __restrict__ blk, int nblk, int E, int T,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ meta, Tile* __restrict__ tiles_s,
                                                     Tile* __restrict__ tiles_w, Tile* __restrict__ tiles_w2) {
  __shared__ int cnt[1024];
  __shared__ int off[1025];
  __shared__ int scratch[8];
  const int per = (E + 255) / 256;
  constexpr int NB = 16;  // token blocks whose counts are loaded together (the loads' latency overlaps)
  // per expert: running base across token blocks (block order = token order)
  for (int j = 0; j < per; ++j) {
    int e = threadIdx.x * per + j;
    if (e >= E) break;
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += NB) {
      int c[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) c[i] = b0 + i < nblk ? blk[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (b0 + i < nblk) blk[(size_t)(b0 + i) * E + e] = run;
        run += c[i];
      }
    }
    cnt[e] = run;
  }
  __syncthreads();
  publish(cnt, off, E, T, counts, offsets, meta, tiles_s, tiles_w, tiles_w2, scratch);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int o = off[e];
    for (int b0 = 0; b0 < nblk; b0 += NB) {
      int c[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) c[i] = b0 + i < nblk ? blk[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (b0 + i < nblk) blk[(size_t)(b0 + i) * E + e] = c[i] + o;
    }
  }
}

__global__ __launch_bounds__(TB) void dispatch_single(const int32_t* __restrict__ idx, int T, int K, int E,
                                                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ meta, Tile* __restrict__ tiles_s,
                                                      Tile* __restrict__ tiles_w, Tile* __restrict__ tiles_w2,
                                                      int32_t* __restrict__ row_token, int32_t* __restrict__ row_of) {
  extern __shared__ unsigned long long bits[];
  __shared__ DispatchLds L;
  dispatch_block(idx, T, K, E, counts, offsets, meta, tiles_s, tiles_w, tiles_w2, row_token, row_of, bits, L);
}

__global__ __launch_bounds__(TB) void dispatch_scatter(const int32_t* __restrict__ idx, int T, int K, int E,
                                                       const int32_t* __restrict__ blk,
                                                       int32_t* __restrict__ row_token, int32_t* __restrict__ row_of) {
  extern __shared__ unsigned long long bits[];
  build_bits(bits, idx, T, K, E, blockIdx.x);
  scatter_rows(bits, idx, T, K, E, blockIdx.x, blk + (size_t)blockIdx.x * E, row_token, row_of);
}

// Tile lists of a dense feed-forward: no routed experts (E = 0), so the lists hold only the
// shared-expert tiles (expert index E) over all T tokens, written by the same code as the
// block's dispatch; offsets[0] = 0 and meta as above.
__global__ __launch_bounds__(TB) void dense_tiles(int T, int32_t* __restrict__ offsets, int32_t* __restrict__ meta,
                                                  Tile* __restrict__ tiles_s, Tile* __restrict__ tiles_w,
                                                  Tile* __restrict__ tiles_w2) {
  __shared__ int cnt[1];
  __shared__ int off[1];
  __shared__ int scratch[8];
  publish(cnt, off, 0, T, nullptr, offsets, meta, tiles_s, tiles_w, tiles_w2, scratch);
}

hipError_t launch_dense_tiles(const Dims& d, int32_t* offsets, int32_t* meta, Tile* tiles_s, Tile* tiles_w,
                              Tile* tiles_w2, hipStream_t s) {
  MOE_LAUNCH(dense_tiles, dim3(1), dim3(TB), 0, s, (int)d.T, offsets, meta, tiles_s, tiles_w, tiles_w2);
  return hipGetLastError();
}

int dispatch_blocks(int64_t T) { return (int)((T + TB - 1) / TB); }

int64_t max_tiles(const Dims& d, int bm) { return d.R / bm + d.E + (d.T + bm - 1) / bm + 1; }

hipError_t launch_dispatch(const Dims& d, const int32_t* idx, int32_t* blk, int32_t* counts, int32_t* offsets,
                           int32_t* row_token, int32_t* row_of, int32_t* meta, Tile* tiles_s, Tile* tiles_w,
                           Tile* tiles_w2, hipStream_t s) {
  int nblk = dispatch_blocks(d.T);
  size_t lds = (size_t)d.E * WORDS * sizeof(unsigned long long);
  if (nblk <= 1) {
    MOE_LAUNCH(dispatch_single, dim3(1), dim3(TB), lds, s, idx, (int)d.T, d.K, d.E, counts, offsets, meta, tiles_s,
               tiles_w, tiles_w2, row_token, row_of);
    return hipGetLastError();
  }
  MOE_LAUNCH(dispatch_count, dim3(nblk), dim3(TB), lds, s, idx, (int)d.T, d.K, d.E, blk);
  MOE_LAUNCH(dispatch_scan, dim3(1), dim3(256), 0, s, blk, nblk, d.E, (int)d.T, counts, offsets, meta, tiles_s,
             tiles_w, tiles_w2);
  MOE_LAUNCH(dispatch_scatter, dim3(nblk), dim3(TB), lds, s, idx, (int)d.T, d.K, d.E, blk, row_token, row_of);
  return hipGetLastError();
}

}  // namespace moe

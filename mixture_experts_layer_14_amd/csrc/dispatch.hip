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
#include "kernels.h"

namespace moe {

constexpr int TB = kDispatchTB;
constexpr int WORDS = TB / 64;

__device__ __forceinline__ void build_bits(unsigned long long* bits, const int32_t* __restrict__ idx, int T, int K,
                                           int E) {
  for (int i = threadIdx.x; i < E * WORDS; i += blockDim.x) bits[i] = 0ull;
  __syncthreads();
  int t = blockIdx.x * TB + threadIdx.x;
  if (t < T) {
    unsigned long long bit = 1ull << (threadIdx.x & 63);
    int w = threadIdx.x >> 6;
    for (int k = 0; k < K; ++k) {
      int e = idx[(size_t)t * K + k];
      if ((unsigned)e < (unsigned)E) atomicOr(&bits[e * WORDS + w], bit);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(TB) void dispatch_count(const int32_t* __restrict__ idx, int T, int K, int E,
                                                     int32_t* __restrict__ blk) {
  extern __shared__ unsigned long long bits[];
  build_bits(bits, idx, T, K, E);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < WORDS; ++w) c += __popcll(bits[e * WORDS + w]);
    blk[(size_t)blockIdx.x * E + e] = c;
  }
}

// Exclusive scan of v over the block (256 threads); returns the block total in *total.
__device__ int block_exclusive_scan(int v, int* scratch /*[4]*/, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < 4; ++w) {
    int sw = scratch[w];
    if (w < wave) before += sw;
    all += sw;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Tiles of one list: routed experts ascending (M-tiles of `bm` dispatch rows), then the
// shared expert (index E) over all T tokens.
__device__ void write_tiles(const int* cnt, const int* off, int E, int T, int bm, Tile* tiles, int32_t* meta_routed,
                            int32_t* meta_all, int* scratch) {
  // each thread owns experts [tid * per, tid * per + per)
  const int per = (E + 255) / 256;
  int mine = 0;
  for (int j = 0; j < per; ++j) {
    int e = threadIdx.x * per + j;
    if (e < E) mine += (cnt[e] + bm - 1) / bm;
  }
  int total;
  int base = block_exclusive_scan(mine, scratch, &total);
  for (int j = 0; j < per; ++j) {
    int e = threadIdx.x * per + j;
    if (e >= E) break;
    int c = cnt[e];
    const int first = base;
    for (int m = 0; m < c; m += bm) {
      Tile tl;
      tl.expert = e;
      tl.row0 = off[e] + m;
      tl.nrows = min(bm, c - m);
      tl.first = first;
      tiles[base++] = tl;
    }
  }
  int nsh = (T + bm - 1) / bm;
  for (int j = threadIdx.x; j < nsh; j += blockDim.x) {
    Tile tl;
    tl.expert = E;
    tl.row0 = j * bm;
    tl.nrows = min(bm, T - j * bm);
    tl.first = total;
    tiles[total + j] = tl;
  }
  if (threadIdx.x == 0) {
    *meta_routed = total;
    *meta_all = total + nsh;
  }
}

// From cnt[E] (LDS): off[0..E] (LDS), counts/offsets, the three tile lists and meta.
__device__ void publish(const int* cnt, int* off, int E, int T, int32_t* __restrict__ counts,
                        int32_t* __restrict__ offsets, int32_t* __restrict__ meta, Tile* __restrict__ tiles_s,
                        Tile* __restrict__ tiles_w, Tile* __restrict__ tiles_w2, int* scratch) {
  const int per = (E + 255) / 256;
  int mine = 0;
  for (int j = 0; j < per; ++j) {
    int e = threadIdx.x * per + j;
    if (e < E) mine += cnt[e];
  }
  int total;
  int base = block_exclusive_scan(mine, scratch, &total);
  int active = 0;
  for (int j = 0; j < per; ++j) {
    int e = threadIdx.x * per + j;
    if (e >= E) break;
    off[e] = base;
    base += cnt[e];
    active += cnt[e] > 0;
  }
  if (threadIdx.x == 0) off[E] = total;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    counts[e] = cnt[e];
    offsets[e] = off[e];
  }
  if (threadIdx.x == 0) offsets[E] = off[E];
  int nact;
  block_exclusive_scan(active, scratch, &nact);
  write_tiles(cnt, off, E, T, kSkinnyBM, tiles_s, &meta[0], &meta[1], scratch);
  __syncthreads();
  write_tiles(cnt, off, E, T, kWideBM, tiles_w, &meta[2], &meta[3], scratch);
  __syncthreads();
  write_tiles(cnt, off, E, T, kWideBM2, tiles_w2, &meta[5], &meta[6], scratch);
  if (threadIdx.x == 0) meta[4] = nact;
  __syncthreads();
}

__global__ __launch_bounds__(256) void dispatch_scan(int32_t* __restrict__ blk, int nblk, int E, int T,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ meta, Tile* __restrict__ tiles_s,
                                                     Tile* __restrict__ tiles_w, Tile* __restrict__ tiles_w2) {
  __shared__ int cnt[1024];
  __shared__ int off[1025];
  __shared__ int scratch[4];
  const int per = (E + 255) / 256;
  // per expert: running base across token blocks (block order = token order)
  for (int j = 0; j < per; ++j) {
    int e = threadIdx.x * per + j;
    if (e >= E) break;
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
      int c = blk[(size_t)b * E + e];
      blk[(size_t)b * E + e] = run;
      run += c;
    }
    cnt[e] = run;
  }
  __syncthreads();
  publish(cnt, off, E, T, counts, offsets, meta, tiles_s, tiles_w, tiles_w2, scratch);
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    for (int b = 0; b < nblk; ++b) blk[(size_t)b * E + e] += off[e];
}

// Row of token t's k-th choice e: base row of e for this token block + earlier tokens of the
// block that chose e (popcount of their bits).
__device__ void scatter_rows(const unsigned long long* bits, const int32_t* __restrict__ idx, int T, int K, int E,
                             const int* base /* [E], this block */, int32_t* __restrict__ row_token,
                             int32_t* __restrict__ row_of) {
  int t = blockIdx.x * TB + threadIdx.x;
  if (t >= T) return;
  const int w = threadIdx.x >> 6;
  const unsigned long long below = (1ull << (threadIdx.x & 63)) - 1ull;
  for (int k = 0; k < K; ++k) {
    int e = idx[(size_t)t * K + k];
    if ((unsigned)e >= (unsigned)E) {  // no row: the combine skips this assignment
      row_of[(size_t)t * K + k] = -1;
      continue;
    }
    int rank = __popcll(bits[e * WORDS + w] & below);
    for (int ww = 0; ww < w; ++ww) rank += __popcll(bits[e * WORDS + ww]);
    int row = base[e] + rank;
    row_token[row] = t;
    row_of[(size_t)t * K + k] = row;
  }
}

// T <= 256: count, scan and scatter in one workgroup.
__global__ __launch_bounds__(TB) void dispatch_single(const int32_t* __restrict__ idx, int T, int K, int E,
                                                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ meta, Tile* __restrict__ tiles_s,
                                                      Tile* __restrict__ tiles_w, Tile* __restrict__ tiles_w2,
                                                      int32_t* __restrict__ row_token, int32_t* __restrict__ row_of) {
  extern __shared__ unsigned long long bits[];
  __shared__ int cnt[1024];
  __shared__ int off[1025];
  __shared__ int scratch[4];
  build_bits(bits, idx, T, K, E);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < WORDS; ++w) c += __popcll(bits[e * WORDS + w]);
    cnt[e] = c;
  }
  __syncthreads();
  publish(cnt, off, E, T, counts, offsets, meta, tiles_s, tiles_w, tiles_w2, scratch);
  scatter_rows(bits, idx, T, K, E, off, row_token, row_of);
}

__global__ __launch_bounds__(TB) void dispatch_scatter(const int32_t* __restrict__ idx, int T, int K, int E,
                                                       const int32_t* __restrict__ blk,
                                                       int32_t* __restrict__ row_token, int32_t* __restrict__ row_of) {
  extern __shared__ unsigned long long bits[];
  build_bits(bits, idx, T, K, E);
  scatter_rows(bits, idx, T, K, E, blk + (size_t)blockIdx.x * E, row_token, row_of);
}

// Tile lists of a dense feed-forward: no routed experts (E = 0), so the lists hold only the
// shared-expert tiles (expert index E) over all T tokens, written by the same code as the
// block's dispatch; offsets[0] = 0 and meta as above.
__global__ __launch_bounds__(TB) void dense_tiles(int T, int32_t* __restrict__ offsets, int32_t* __restrict__ meta,
                                                  Tile* __restrict__ tiles_s, Tile* __restrict__ tiles_w,
                                                  Tile* __restrict__ tiles_w2) {
  __shared__ int cnt[1];
  __shared__ int off[1];
  __shared__ int scratch[4];
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

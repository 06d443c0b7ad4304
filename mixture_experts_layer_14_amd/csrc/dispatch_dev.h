// Device code of the dispatch shared by its kernels and the fused decode kernel ("DeepSeek-V3.2-Exp ·
// Mixture of experts", MoE.forward excerpt: bincount, then each expert's tokens in token order).
#pragma once
#include "kernels.h"

namespace moe {

constexpr int TB = kDispatchTB;
constexpr int WORDS = TB / 64;

// LDS of a single-workgroup dispatch (besides the token bitmap)
struct DispatchLds {
  int cnt[1024];
  int off[1025];
  int scratch[8];
};

// Bitmap of token block `tb` (tokens tb * TB ..): bit (e, t) set when token t chose e. Threads past
// the first TB only clear and synchronise.
__device__ __forceinline__ void build_bits(unsigned long long* bits, const int32_t* __restrict__ idx, int T, int K,
                                           int E, int tb) {
  for (int i = threadIdx.x; i < E * WORDS; i += blockDim.x) bits[i] = 0ull;
  __syncthreads();
  int t = tb * TB + threadIdx.x;
  if (threadIdx.x < TB && t < T) {
    unsigned long long bit = 1ull << (threadIdx.x & 63);
    int w = threadIdx.x >> 6;
    for (int k = 0; k < K; ++k) {
      int e = idx[(size_t)t * K + k];
      if ((unsigned)e < (unsigned)E) atomicOr(&bits[e * WORDS + w], bit);
    }
  }
  __syncthreads();
}

// Tiles of one list: routed experts ascending (M-tiles of `bm` dispatch rows), then the
// shared expert (index E) over all T tokens.
MOE_DEV void write_tiles(const int* cnt, const int* off, int E, int T, int bm, Tile* tiles, int32_t* meta_routed,
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
MOE_DEV void publish(const int* cnt, int* off, int E, int T, int32_t* __restrict__ counts,
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

// Row of token t's k-th choice e: base row of e for this token block + earlier tokens of the
// block that chose e (popcount of their bits).
MOE_DEV void scatter_rows(const unsigned long long* bits, const int32_t* __restrict__ idx, int T, int K, int E,
                             int tb, const int* base /* [E], this block */, int32_t* __restrict__ row_token,
                             int32_t* __restrict__ row_of) {
  int t = tb * TB + threadIdx.x;
  if (threadIdx.x >= TB || t >= T) return;
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

// T <= 256: count, scan and scatter in one workgroup of 256 or 512 threads. bits: E * TB / 64 words
// of LDS.
MOE_DEV void dispatch_block(const int32_t* __restrict__ idx, int T, int K, int E, int32_t* __restrict__ counts,
                            int32_t* __restrict__ offsets, int32_t* __restrict__ meta, Tile* __restrict__ tiles_s,
                            Tile* __restrict__ tiles_w, Tile* __restrict__ tiles_w2, int32_t* __restrict__ row_token,
                            int32_t* __restrict__ row_of, unsigned long long* bits, DispatchLds& L) {
  build_bits(bits, idx, T, K, E, 0);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < WORDS; ++w) c += __popcll(bits[e * WORDS + w]);
    L.cnt[e] = c;
  }
  __syncthreads();
  publish(L.cnt, L.off, E, T, counts, offsets, meta, tiles_s, tiles_w, tiles_w2, L.scratch);
  scatter_rows(bits, idx, T, K, E, 0, L.off, row_token, row_of);
}

}  // namespace moe

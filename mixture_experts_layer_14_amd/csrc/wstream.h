// Device helpers shared by the per-wave weight-stream GEMM kernels (bf16 and fp8 prefill).
#pragma once
#include "ring.h"

namespace moe {

constexpr int WS_OOB = 0x7fffffff;    // buffer offset past every range: the load returns zeros
constexpr int WS_RANGE = 0x7ffffff0;  // byte range of the activation resources (tensors < 2 GB)

// LDS rows of 128 bytes (8 chunks of 16 bytes): chunk c of row r sits at slot c ^ key(r), with
// key(r) = (r & 7) ^ ((r >> 3) & 3), a function of r mod 32 only. Any 8 consecutive rows, and
// the even and the odd rows of 16 consecutive rows, use 8 distinct slots, so a fragment read (32
// consecutive rows, one chunk) is free of bank conflicts; and because the key repeats every 32
// rows, the fragment address of every 32-row group is one per-lane base plus a constant. A load
// instruction fills 8 consecutive rows 8 i .. 8 i + 7 (lane: row 8 i + lane / 8, slot lane % 8),
// so the lane fetches chunk (lane % 8) ^ (lane / 8) ^ (i % 4).
MOE_DEV int ws_key(int row) { return (row & 7) ^ ((row >> 3) & 3); }
MOE_DEV int ws_pos(int row, int chunk) { return row * 128 + ((chunk ^ ws_key(row)) << 4); }

MOE_DEV __amdgpu_buffer_rsrc_t ws_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

template <bool NT>
MOE_DEV void ws_dma(__amdgpu_buffer_rsrc_t r, char* lds_dst, int voff, int soff) {
  constexpr int AUX = NT ? 2 : 0;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, voff, soff, 0, AUX);
}

// Runs of kRunBlocks blocks. A run is a contiguous range [lo, hi) of whole tiles of a tile list
// holding an equal share of the launch's cost: cost(t) is tile t's cost, item(t) the list index of
// its first item (item(ntiles) = items), and a bound is the tile boundary nearest to its share.
// Every thread of the block calls it; red: 10 ints of LDS that no load is writing. Returns whether
// the run has items.
constexpr int kRunBlocks = 16;
template <class Cost, class Item>
MOE_DEV bool ws_run_bounds(int ntiles, int items, int run, int nruns, Cost cost, Item item, int* red, int& lo,
                           int& hi) {
  const int per_t = (ntiles + (int)blockDim.x - 1) / (int)blockDim.x;
  const int t0 = min(ntiles, (int)threadIdx.x * per_t), t1 = min(ntiles, t0 + per_t);
  int mine = 0;
  for (int t = t0; t < t1; ++t) mine += cost(t);
  int total = 0;
  const int before = block_exclusive_scan(mine, red, &total);
  if (threadIdx.x == 0) {
    red[8] = run == 0 ? 0 : -1;
    red[9] = run + 1 == nruns ? items : -1;
  }
  __syncthreads();
  for (int b = 0; b < 2; ++b) {
    const int r = run + b;
    if (r == 0 || r == nruns) continue;
    const int64_t target = (int64_t)total * r / nruns;
    int acc = before;
    for (int t = t0; t < t1; ++t) {  // one thread's range holds the target
      const int c = cost(t);
      if (acc <= target && target < acc + c) red[8 + b] = item(2 * (target - acc) < c ? t : t + 1);
      acc += c;
    }
  }
  __syncthreads();
  lo = red[8];
  hi = red[9];
  __syncthreads();  // every bound is read before the LDS is written again
  return total > 0 && lo >= 0 && hi > lo;  // with no tiles there is no work (and no bound)
}

// A run's blocks take its items in rounds of kRunBlocks consecutive ones, the block's place in the
// round (pos) moving by one each round: ws_run_count items, the i-th at ws_run_item.
MOE_DEV int ws_run_count(int lo, int hi, int pos) {
  const int q = (hi - lo) / kRunBlocks, rest = (hi - lo) % kRunBlocks;
  return q + ((pos + q) % kRunBlocks < rest ? 1 : 0);
}
MOE_DEV int ws_run_item(int lo, int pos, int i) { return lo + kRunBlocks * i + (pos + i) % kRunBlocks; }

struct WsItem {  // one work item of a block (wave-uniform)
  int row0, nrows, nt, expert, rot;
  bool sh, live;
  bool solo;  // the item's expert has a single M-tile: no other item reads its weight tiles
};

}  // namespace moe

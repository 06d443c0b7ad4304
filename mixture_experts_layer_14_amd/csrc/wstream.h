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

struct WsItem {  // one work item of a block (wave-uniform)
  int row0, nrows, nt, expert, rot;
  bool sh, live;
  bool solo;  // the item's expert has a single M-tile: no other item reads its weight tiles
};

}  // namespace moe

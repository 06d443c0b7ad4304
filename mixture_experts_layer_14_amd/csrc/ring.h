// Device helpers of the direct global->LDS ring kernel (bf16 prefill GEMMs).
#pragma once
#include "kernels.h"

namespace moe {

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their no-wait maxima).
template <int N>
MOE_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// wait until at most n (0..63) vector-memory operations of this wave are outstanding
MOE_DEV void wait_vmcnt_upto(int n) {
#define MOE_VMW(v) \
  case v: wait_vmcnt<v>(); return;
  switch (n) {
    MOE_VMW(0) MOE_VMW(1) MOE_VMW(2) MOE_VMW(3) MOE_VMW(4) MOE_VMW(5) MOE_VMW(6) MOE_VMW(7)
    MOE_VMW(8) MOE_VMW(9) MOE_VMW(10) MOE_VMW(11) MOE_VMW(12) MOE_VMW(13) MOE_VMW(14) MOE_VMW(15)
    MOE_VMW(16) MOE_VMW(17) MOE_VMW(18) MOE_VMW(19) MOE_VMW(20) MOE_VMW(21) MOE_VMW(22) MOE_VMW(23)
    MOE_VMW(24) MOE_VMW(25) MOE_VMW(26) MOE_VMW(27) MOE_VMW(28) MOE_VMW(29) MOE_VMW(30) MOE_VMW(31)
    MOE_VMW(32) MOE_VMW(33) MOE_VMW(34) MOE_VMW(35) MOE_VMW(36) MOE_VMW(37) MOE_VMW(38) MOE_VMW(39)
    MOE_VMW(40) MOE_VMW(41) MOE_VMW(42) MOE_VMW(43) MOE_VMW(44) MOE_VMW(45) MOE_VMW(46) MOE_VMW(47)
    default: wait_vmcnt<0>(); return;
  }
#undef MOE_VMW
}
// s_waitcnt lgkmcnt(0): this wave's LDS reads have returned.
MOE_DEV void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

MOE_DEV void barrier_only() { __builtin_amdgcn_s_barrier(); }

// 16 bytes per lane from global memory straight into LDS (lane i -> lds_wave_base + 16 i).
MOE_DEV void lds_dma16(const void* g, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
// the same with the nontemporal hint, for data read once
MOE_DEV void lds_dma16_nt(const void* g, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 2);
}

// LDS row layout of a stage: rows of BK bf16 = ROWB bytes = CPR 16-byte chunks; chunk c of
// row r sits at position c ^ key(r). For 8 chunks per row, key(r) = (r ^ (r >> 3)) & 7 (as
// swz()); for 4, key(r) = ((r >> 1) ^ (r >> 3)) & 3. Either way the rows read together by
// one fragment load (32 consecutive rows, one chunk) spread over all banks whether the LDS
// serves 8 or 16 lanes of 16 bytes per cycle.
template <int CPR>
MOE_DEV int ring_key(int row) {
  return CPR == 8 ? ((row ^ (row >> 3)) & 7) : (((row >> 1) ^ (row >> 3)) & 3);
}
template <int CPR>
MOE_DEV int ring_pos(int row, int chunk) {
  return row * (CPR * 16) + ((chunk ^ ring_key<CPR>(row)) << 4);
}

}  // namespace moe

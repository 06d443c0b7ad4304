// Router of the MoE block ("DeepSeek-V3.2-Exp · Router", formula steps 1-4 and the
// Gate.forward excerpt): logits, sigmoid, selection bias, group-limited top-k,
// renormalised and scaled weights.
#include <float.h>
#include <math.h>

#include <algorithm>

#include "router_dev.h"
#include "wstream.h"

namespace moe {

// Block: 4 waves on one tile of 32 tokens x 32 experts (logits_tile). Grid (T/32, E/32, nsplit).
__global__ __launch_bounds__(256) void router_logits_bf16(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wg,
                                                          double* __restrict__ zpart, int T, int D, int E,
                                                          int kslice) {
  __shared__ double red[3][16][64];
  logits_tile(x, wg, zpart, T, D, E, kslice, blockIdx.x, blockIdx.y, blockIdx.z, red);
}

// Large batches: a block holds 64 tokens x 256 experts over one k-slice, so x is read once per
// slice and W_r once per 64 tokens. Both operands go global -> LDS directly in 64-k stages (64 x
// rows and 256 W_r rows of 128 bytes, in the XOR layout of ws_pos), three stages in a ring whose
// loads run two stages ahead of the MFMAs. Wave w (of 8) takes tokens 32 (w / 4) .. + 31 and
// experts 64 (w % 4) .. + 63 and adds its 32-k chunk sums in k order. Grid (T/64, E/256, nsplit).
constexpr int RW_X = 64 * 128;              // x rows of a stage (bytes)
constexpr int RW_STAGE = RW_X + 256 * 128;  // x rows, then W_r rows
constexpr int RW_NS = 3;
constexpr size_t RW_LDS = (size_t)RW_NS * RW_STAGE;

__global__ __launch_bounds__(512) void router_logits_bf16_wide(const bf16_t* __restrict__ x,
                                                               const bf16_t* __restrict__ wg,
                                                               double* __restrict__ zpart, int T, int D, int E,
                                                               int kslice) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int split = blockIdx.z;
  const int kb = split * kslice, ke = min(D, kb + kslice);
  const int nch = max(0, ke - kb) / 32;  // 32-k chunks of the slice
  const int ns = (nch + 1) / 2;          // 64-k stages
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 256;
  const int nt = min(64, T - t0), ne = min(256, E - e0);

  // Loads: one instruction fills 8 stage rows (lane: row + lane / 8, slot lane % 8, fetching the
  // chunk that belongs in that slot). This wave fills x rows 8 w .. and W_r rows 8 (w + 8 j) ..;
  // a lane whose row lies past the tile, or whose chunk lies past the slice, reads zeros.
  const __amdgpu_buffer_rsrc_t rx = ws_rsrc(x + (size_t)t0 * D, nt * D * 2);
  const __amdgpu_buffer_rsrc_t rw = ws_rsrc(wg + (size_t)e0 * D, ne * D * 2);
  const int xrow = wave * 8 + (lane >> 3);
  const int xc = (lane & 7) ^ ws_key(xrow);
  const int xoff = xrow < nt ? xrow * D * 2 + xc * 16 : WS_OOB;
  int woff[4], wc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (wave + 8 * j) * 8 + (lane >> 3);
    wc[j] = (lane & 7) ^ ws_key(row);
    woff[j] = row < ne ? row * D * 2 + wc[j] * 16 : WS_OOB;
  }
  auto issue = [&](int st) __attribute__((always_inline)) {
    char* dst = lds + (st % RW_NS) * RW_STAGE;
    const int kbyte = (kb + 64 * st) * 2;
    const int c0 = 2 * st;  // the stage's first chunk; a lane's 16 bytes are in chunk c0 + (slot chunk >= 4)
    ws_dma<false>(rx, dst + wave * 1024, c0 + (xc >> 2) < nch ? xoff : WS_OOB, kbyte);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      ws_dma<false>(rw, dst + RW_X + (wave + 8 * j) * 1024, c0 + (wc[j] >> 2) < nch ? woff[j] : WS_OOB, kbyte);
  };
  constexpr int kLoads = 5;  // per thread and stage

  // fragments: A (tokens) and B (experts) rows of 16, the 16 bytes of chunk 4 c + lane / 16
  const int r = lane & 15, kq = lane >> 4;
  const int tw = (wave >> 2) * 32, ew = (wave & 3) * 64;
  int fa[2][2], fb[4][2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int m = 0; m < 2; ++m) fa[m][c] = ws_pos(tw + m * 16 + r, 4 * c + kq);
#pragma unroll
    for (int n = 0; n < 4; ++n) fb[n][c] = RW_X + ws_pos(ew + n * 16 + r, 4 * c + kq);
  }
  double acc[2][4][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][n][i] = 0.0;
  const f32x4 fz = {0.f, 0.f, 0.f, 0.f};

  // fragments of one stage: a[c][m] tokens, b[c][n] experts of chunk c
  struct Frag {
    i32x4 a[2][2], b[2][4];
  };
  auto read = [&](Frag& f, int st) __attribute__((always_inline)) {
    const char* sl = lds + (st % RW_NS) * RW_STAGE;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int m = 0; m < 2; ++m) f.a[c][m] = *reinterpret_cast<const i32x4*>(sl + fa[m][c]);
#pragma unroll
      for (int n = 0; n < 4; ++n) f.b[c][n] = *reinterpret_cast<const i32x4*>(sl + fb[n][c]);
    }
  };
  // acc += chunk sums of stage st, chunk 0 then chunk 1 (k order). The MFMAs of chunk 1 go out
  // between the fp64 additions of chunk 0, each result in registers of its own, so the matrix
  // core works while the additions run.
  auto add = [&](const f32x4& p, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j >> 2][j & 3][i] += (double)p[i];
  };
  auto multiply = [&](const Frag& f, int st) __attribute__((always_inline)) {
    f32x4 p0[8], p1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p0[j] = mfma_bf16_16x16x32(f.a[0][j >> 2], f.b[0][j & 3], fz);
    if (2 * st + 1 < nch) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p1[j] = mfma_bf16_16x16x32(f.a[1][j >> 2], f.b[1][j & 3], fz);
        add(p0[j], j);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // VALU
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) add(p1[j], j);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) add(p0[j], j);
    }
  };

  issue(0);
  issue(1);
  Frag f;
  for (int st = 0; st < ns; ++st) {
    wait_vmcnt<kLoads>();  // this thread's loads of stage st have landed (those of st + 1 may not)
    barrier_only();        // everyone's have; everyone is done reading stage st - 1
    issue(st + 2);         // into the slot of stage st - 1
    read(f, st);
    multiply(f, st);
  }
  wait_vmcnt<0>();  // the loads issued past the last stage (zeros) have landed before the wave ends
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int e = e0 + ew + n * 16 + r;
      if (e >= E) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + tw + m * 16 + kq * 4 + i;
        if (t < T) zpart[((size_t)split * T + t) * E + e] = acc[m][n][i];
      }
    }
}

// fp32 inputs: each product is exact in fp64; one thread per (token, expert).
__global__ __launch_bounds__(256) void router_logits_f32(const float* __restrict__ x, const float* __restrict__ wg,
                                                         double* __restrict__ zpart, int T, int D, int E) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * E) return;
  int t = (int)(i / E), e = (int)(i % E);
  const float* xr = x + (size_t)t * D;
  const float* wr = wg + (size_t)e * D;
  double acc = 0.0;
  for (int k = 0; k < D; ++k) acc += (double)xr[k] * (double)wr[k];
  zpart[i] = acc;
}

template <int EPT, int TPB>
__global__ __launch_bounds__(256) void router_select(const double* __restrict__ zpart, int nsplit,
                                                     const float* __restrict__ bias, int T, int E, int G, int Gk,
                                                     int K, float route_scale, int softmax,
                                                     int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  __shared__ SelectLds<EPT, TPB, 256 / TPB> L;
  select_block<EPT, TPB, 256>(blockIdx.x, zpart, nsplit, bias, T, E, G, Gk, K, route_scale, softmax, idx_out, w_out, L);
}

// Batches of 1024 tokens or more use the 64 x 256 tiles.
static bool router_wide(const Dims& d) { return d.dtype != 0 && d.T >= 1024; }

int router_splits(const Dims& d) {
  if (d.dtype == 0 || d.T == 0) return 1;
  const bool wide = router_wide(d);
  int64_t tiles = wide ? ((d.T + 63) / 64) * ((d.E + 255) / 256) : ((d.T + 31) / 32) * ((d.E + 31) / 32);
  // enough blocks to stream the router weight with many CUs, but few slices to add up, each
  // at least one chunk per wave
  int64_t want = (256 + tiles - 1) / tiles;
  int64_t max_split = std::min<int64_t>(kMaxSplit, d.D / (wide ? 64 : 128));
  if (want > max_split) want = max_split;
  if (want < 1) want = 1;
  return (int)want;
}

int router_kslice(const Dims& d, int nsplit) {
  int chunks = d.D / 32;
  return ((chunks + nsplit - 1) / nsplit) * 32;
}

hipError_t launch_router_logits(const Dims& d, const void* x, const void* w_gate, double* zpart, int nsplit,
                                hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  if (d.dtype == 0) {
    int64_t n = d.T * d.E;
    MOE_LAUNCH(router_logits_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float*)x, (const float*)w_gate, zpart, (int)d.T, d.D, d.E);
  } else {
    const int kslice = router_kslice(d, nsplit);
    // the 64 x 256 tiles where the device gives a block the LDS of their ring; the 32 x 32 tiles
    // take the same slices otherwise
    if (router_wide(d) && device_lds_limit() >= (int)RW_LDS) {
      dim3 grid((unsigned)((d.T + 63) / 64), (unsigned)((d.E + 255) / 256), (unsigned)nsplit);
      hipError_t e = allow_dynamic_lds((const void*)router_logits_bf16_wide, RW_LDS);
      if (e != hipSuccess) return e;
      MOE_LAUNCH(router_logits_bf16_wide, grid, dim3(512), RW_LDS, s, (const bf16_t*)x, (const bf16_t*)w_gate, zpart,
                 (int)d.T, d.D, d.E, kslice);
    } else {
      dim3 grid((unsigned)((d.T + 31) / 32), (unsigned)((d.E + 31) / 32), (unsigned)nsplit);
      MOE_LAUNCH(router_logits_bf16, grid, dim3(256), 0, s, (const bf16_t*)x, (const bf16_t*)w_gate, zpart,
                 (int)d.T, d.D, d.E, kslice);
    }
  }
  return hipGetLastError();
}

hipError_t launch_router_select(const Dims& d, const double* zpart, int nsplit, const float* bias,
                                float route_scale, bool softmax, int32_t* idx, float* w, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  // the selection kernel's per-token arrays are sized for these limits (the ABI rejects larger
  // configurations before any launch)
  if (d.E > kMaxE || d.G > kMaxG || d.K > kMaxK || nsplit > kMaxSplit) return hipErrorInvalidValue;
  // one token per block for small batches (latency), one per wave for large ones with E <= 256
#define MOE_SELECT(EPT, TPB)                                                                              \
  MOE_LAUNCH((router_select<EPT, TPB>), dim3((unsigned)((d.T + TPB - 1) / TPB)), dim3(256), 0, s, zpart, nsplit, \
             bias, (int)d.T, d.E, d.G, d.Gk, d.K, route_scale, softmax ? 1 : 0, idx, w)
  if (d.T > 256 && d.E <= 64) MOE_SELECT(1, 4);
  else if (d.T > 256 && d.E <= 128) MOE_SELECT(2, 4);
  else if (d.T > 256 && d.E <= 256) MOE_SELECT(4, 4);
  else if (d.E <= 256) MOE_SELECT(1, 1);
  else if (d.E <= 512) MOE_SELECT(2, 1);
  else MOE_SELECT(4, 1);
#undef MOE_SELECT
  return hipGetLastError();
}

}  // namespace moe

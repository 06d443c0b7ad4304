// Host-side launchers of the libmoe kernels (internal; the public ABI is include/moe.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace moe {

// Measurement spans: when timing is enabled (moe_timing_enable), each kernel launch whose name
// passes the filter (moe_timing_filter) is bracketed by HIP events on its stream; otherwise these
// do nothing. span_begin returns whether it recorded.
bool span_begin(const char* name, hipStream_t s);
void span_end(hipStream_t s);
struct Span {
  hipStream_t s;
  bool on;
  Span(const char* name, hipStream_t st) : s(st), on(span_begin(name, st)) {}
  ~Span() {
    if (on) span_end(s);
  }
};
// Launch `kernel` on stream `s` (a variable in scope) inside a measurement span.
#define MOE_LAUNCH(kernel, ...)                         \
  do {                                                  \
    ::moe::Span sp_(#kernel, s);                        \
    hipLaunchKernelGGL(kernel, __VA_ARGS__);            \
  } while (0)

// Rows per M-tile of the tile lists the dispatch writes.
constexpr int kSkinnyBM = 16;
constexpr int kWideBM = 128;
constexpr int kWideBM2 = 256;
constexpr int kDispatchTB = 256;  // tokens per dispatch block

// meta[] written by dispatch_scan (int32):
//   [0] routed tiles (BM 16)   [1] all tiles (BM 16)
//   [2] routed tiles (BM 128)  [3] all tiles (BM 128)
//   [4] experts with tokens
//   [5] routed tiles (BM 256)  [6] all tiles (BM 256)
constexpr int kMetaInts = 8;

struct Dims {
  int64_t T, R;            // tokens, routed rows (T * K)
  int D, E, G, Gk, K, I, S;
  int dtype;               // moe_dtype
};

// ---- router
int router_splits(const Dims& d);
hipError_t launch_router_logits(const Dims& d, const void* x, const void* w_gate, double* zpart, int nsplit,
                                hipStream_t s);
// Sums the nsplit slices of zpart per token in slice order, then scores (sigmoid, or softmax over
// the token's experts), groups and selects.
hipError_t launch_router_select(const Dims& d, const double* zpart, int nsplit, const float* bias,
                                float route_scale, bool softmax, int32_t* idx, float* w, hipStream_t s);

// ---- dispatch
int dispatch_blocks(int64_t T);
// The tile lists and meta of a dense feed-forward (E = 0: only shared-expert tiles over T tokens).
hipError_t launch_dense_tiles(const Dims& d, int32_t* offsets, int32_t* meta, Tile* tiles_s, Tile* tiles_w,
                              Tile* tiles_w2, hipStream_t s);
hipError_t launch_dispatch(const Dims& d, const int32_t* idx, int32_t* blk, int32_t* counts, int32_t* offsets,
                           int32_t* row_token, int32_t* row_of, int32_t* meta, Tile* tiles_skinny,
                           Tile* tiles_wide, Tile* tiles_wide2, hipStream_t s);
int64_t max_tiles(const Dims& d, int bm);

// ---- fp8 activation quantisation (x -> e4m3 + per 1x128 scales)
hipError_t launch_act_quant(const Dims& d, const bf16_t* x, uint8_t* xq, float* sx, hipStream_t s);

// ---- expert GEMMs
struct ExpertPtrs {
  const void *w1, *w3, *w2, *ws1, *ws3, *ws2;
  const float *s1, *s3, *s2, *ss1, *ss3, *ss2;
};
struct Act {
  const void* x;            // [T, D] x (f32 / bf16) or xq (e4m3)
  const float* x_scale;     // fp8: [T, D/128]
  const int32_t* row_token; // [R]
  const int32_t* offsets;   // [E + 1]
  const int32_t* meta;
  const Tile* tiles_skinny;
  const Tile* tiles_wide;    // 128-row M-tiles
  const Tile* tiles_wide2;   // 256-row M-tiles
  void* h_routed;           // [R, I]
  void* h_shared;           // [T, S]
  float* h_scale;           // fp8: [R, I/128]
  float* h_shared_scale;    // fp8: [T, S/128]
  void* o_routed;           // [R, D]
  void* o_shared;           // [T, D]
  float* part = nullptr;    // [split, T, D] fp32 partial sums of a k-split down projection
};
hipError_t launch_experts(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s);
// 16-row weight-streaming bf16 kernels (decode-sized batches)
hipError_t launch_stream_bf16(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s);
// Dense feed-forward (E = 0): tokens from which the 128-row kernels take over, and the k split of
// the 16-row down projection below that (1 = none; > 1 needs Act::part of split * T * D floats).
constexpr int64_t kDenseWideRows = 64;
int dense_down_split(const Dims& d);
// Blocks of `kernel` that fit on the current device at once (occupancy x CUs, the occupancy capped
// at max_per_cu when that is positive), cached per device and kernel.
int persistent_grid(const void* kernel, int threads, size_t dyn_lds = 0, int max_per_cu = 0);
// The current device's per-block LDS limit (cached per device).
int device_lds_limit();
// Once per (device, kernel): let `kernel` take `bytes` of dynamic LDS; the result is cached.
hipError_t allow_dynamic_lds(const void* kernel, size_t bytes);
// 128-row LDS-tiled fp8 kernels with 128-k scale promotion (prefill-sized batches)
bool wide_fp8_ok(const Dims& d);
hipError_t launch_wide_fp8(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s);
// 256-row bf16 kernels fed by a direct-to-LDS 3-stage ring (dim % 128, inter % 64)
bool ring_ok(const Dims& d);

hipError_t launch_ring_bf16(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s);
// 256-row bf16 kernels with a weight stream per wave and a shared activation ring (dim % 256,
// inter % 128)
bool wstream_ok(const Dims& d);
hipError_t launch_wstream_bf16(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s);
// the fp8 counterpart: 128-k scale-block steps, 8 waves of 32 weight rows (dim % 512, inter % 512)
bool wstream_fp8_ok(const Dims& d);
hipError_t launch_wstream_fp8(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s);
// 128-row LDS-tiled bf16 kernels (prefill-sized batches)
bool wide_ok(const Dims& d);
hipError_t launch_wide_bf16(const Dims& d, const ExpertPtrs& w, const Act& a, hipStream_t s);

// ---- the fused single-launch decode (bf16, at most kFusedMaxT tokens and kFusedMaxE experts)
constexpr int kFusedMaxT = 32;
constexpr int kFusedMaxE = 256;
bool decode_fused_ok(const Dims& d);
// Router logits' k-slice length for nsplit slices (whole 32-element chunks).
int router_kslice(const Dims& d, int nsplit);
hipError_t launch_decode_fused(const Dims& d, const ExpertPtrs& w, const void* w_gate, const float* bias,
                               float route_scale, bool softmax, const void* x, double* zpart, int nsplit, int32_t* idx,
                               float* wt, int32_t* counts, const Act& a, int32_t* row_of, void* out, hipStream_t s);

// ---- combine
hipError_t launch_combine(const Dims& d, const int32_t* idx, const float* w, const int32_t* row_of,
                          const void* o_routed, const void* o_shared, void* out, hipStream_t s);

// ---- device helpers shared by the 128-row (wide) kernels
// LDS tile rows are 128 bytes (8 chunks of 16 bytes). Chunk c of row r sits at position
// c ^ f(r), f(r) = (r ^ (r >> 3)) & 7: any 8 consecutive rows, and the even and the odd rows
// of any 16 consecutive rows, use 8 distinct positions, so a 16-byte-per-lane fragment read
// of one chunk over consecutive rows is free of bank conflicts.
MOE_DEV int swz_key(int row) { return (row ^ (row >> 3)) & 7; }
MOE_DEV int swz(int row, int chunk) { return row * 128 + ((chunk ^ swz_key(row)) << 4); }

struct WideItem {
  Tile tl;
  int nt;
  int mt;  // m-tiles of the item's expert (how often its weight tiles are read)
  bool shared;
};

// Exclusive scan of v over the block (blockDim.x threads, at most 8 waves); returns the block total
// in *total. scratch: 8 ints of LDS.
MOE_DEV int block_exclusive_scan(int v, int* scratch, int* total) {
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
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    int sw = scratch[w];
    if (w < wave) before += sw;
    all += sw;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// item -> (tile, n-tile): routed items first (per_r n-tiles per expert), then the shared
// expert's (per_s). Within an expert the M-tiles go in round(mt / kGroupM) groups of nearly equal
// size (the first mt % groups one larger); a group's items run n-tile by n-tile, its M-tiles
// adjacent within an n-tile. Blocks that run together on one XCD (32 consecutive items) then
// share each weight tile among the group's M-tiles and each activation tile among the n-tiles in
// flight. With G M-tiles per group an expert's operand traffic goes as weights / G +
// activations * G / 32, weight tiles being twice the bytes of an activation tile: least at
// G = 8 (a large expert then moves 256 KB of distinct operands per k-step instead of 544 KB for
// 32 M-tiles of one n-tile), within 4% for 6 to 11. An expert of up to 11 M-tiles stays one group
// in the plain order.
constexpr int kGroupM = 8;
template <int BM = kWideBM>
MOE_DEV WideItem wide_item(int item, const Tile* __restrict__ tiles, int nr, const int32_t* __restrict__ offsets,
                           int T, int E, int per_r, int per_s) {
  int per = per_r, base_tiles = 0, local_item = item;
  if (item >= nr * per_r) {
    per = per_s;
    base_tiles = nr;
    local_item = item - nr * per_r;
  }
  // the tile with index item / per belongs to the right expert: each expert owns
  // (its m-tiles) x per consecutive items
  const Tile probe = tiles[base_tiles + local_item / per];
  const int first = probe.first;
  const int rows = probe.expert == E ? T : offsets[probe.expert + 1] - offsets[probe.expert];
  const int mt = (rows + BM - 1) / BM;
  const int local = local_item - (first - base_tiles) * per;
  const int ng = max(1, (mt + kGroupM / 2) / kGroupM);
  const int base = mt / ng, big = mt % ng;  // groups 0 .. big-1 hold base + 1 M-tiles, the rest base
  const int split = big * (base + 1) * per;  // first item of the smaller groups
  int g, gsz, rem;
  if (local < split) {
    gsz = base + 1;
    g = local / (gsz * per);
    rem = local - g * gsz * per;
  } else {
    gsz = base;
    g = big + (local - split) / (gsz * per);
    rem = local - split - (g - big) * gsz * per;
  }
  const int m0 = g * base + min(g, big);  // the group's first M-tile
  WideItem w;
  w.nt = rem / gsz;
  w.mt = mt;
  w.tl = tiles[first + m0 + rem % gsz];
  w.shared = probe.expert == E;
  return w;
}

}  // namespace moe

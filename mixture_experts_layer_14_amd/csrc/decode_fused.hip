// The whole MoE block for decode-sized bf16 batches in one cooperative launch: router logits,
// selection + dispatch, gate/up + SwiGLU, down projection and combine run as five phases of one
// persistent grid, separated by grid-wide barriers ("DeepSeek-V3.2-Exp · Router", formula steps 1-4;
// "DeepSeek-V3.2-Exp · Mixture of experts", MoE.forward excerpt). Decode is bound by reading the
// touched experts' weights once ("Hardware for DeepSeek-V3 and R1", per-token speed follows the
// bytes read), so what a single launch can save is the launch gaps and the tail of each small
// kernel between the two weight streams.
//
// Each phase runs the same device code as the separate kernels of moe_forward, so the result is
// the same bit for bit: the router tiles of router_logits_bf16 (waves 0-3 of a block), the
// wave-per-token selection and the single-workgroup dispatch (both on block 0), the
// 16-row stream GEMMs (gate/up on 8-wave blocks splitting dim; the down projection with each of
// the 8 waves on its own items) and the combine (a token per block). One block per CU: the
// gate/up phase sets the register budget (two waves per SIMD), as in its own kernel.
#include <hip/hip_cooperative_groups.h>

#include "combine_dev.h"
#include "dispatch_dev.h"
#include "router_dev.h"
#include "stream_dev.h"

namespace moe {

namespace cg = cooperative_groups;

constexpr int FD_THREADS = 512;
constexpr int FD_TOKENS = 8;  // selection: tokens per block, a wave each

struct FusedArgs {
  const bf16_t *x, *w_gate;
  const float* bias;
  const bf16_t *w1, *w3, *w2, *ws1, *ws3, *ws2;
  double* zpart;
  int32_t *idx, *counts, *offsets, *row_token, *row_of, *meta;
  float* w;
  Tile *tiles_s, *tiles_w, *tiles_w2;
  bf16_t *h_routed, *h_shared, *o_routed, *o_shared, *out;
  int T, D, E, G, Gk, K, I, S, nsplit, kslice, softmax;
  float route_scale;
};

// LDS of the phases, one at a time
union FusedLds {
  double red[3][16][64];
  SelectLds<4, FD_TOKENS, FD_THREADS / FD_TOKENS> sel;
  struct {
    unsigned long long bits[kFusedMaxE * WORDS];
    DispatchLds d;
  } disp;
  char g1[G1_WAVES][2 * SLAB];
  char g2[FD_THREADS / 64][SLAB];
  struct {
    int srow[kMaxTopK];
    float sw[kMaxTopK];
  } comb;
};

__global__ __launch_bounds__(FD_THREADS) void decode_fused(FusedArgs a) {
  __shared__ FusedLds L;
  cg::grid_group grid = cg::this_grid();
  const int bid = blockIdx.x, nb = gridDim.x;

  // router logits: tiles (0, by, split) of 32 tokens x 32 experts x one k-slice
  const int gy = (a.E + 31) / 32;
  for (int u = bid; u < gy * a.nsplit; u += nb) {
    logits_tile(a.x, a.w_gate, a.zpart, a.T, a.D, a.E, a.kslice, 0, u % gy, u / gy, L.red);
    __syncthreads();  // red is reused by the block's next tile
  }
  grid.sync();

  // selection (a wave per token) and dispatch, both on block 0: a grid barrier between them cost
  // more than the selection's parallelism across blocks saved (measured 38 + 26 us as two phases)
  if (bid == 0) {
    for (int b = 0; b * FD_TOKENS < a.T; ++b) {
      select_block<4, FD_TOKENS, FD_THREADS>(b, a.zpart, a.nsplit, a.bias, a.T, a.E, a.G, a.Gk, a.K, a.route_scale,
                                             a.softmax, a.idx, a.w, L.sel);
      __syncthreads();  // this block's idx and w are written before dispatch reads them
    }
    dispatch_block(a.idx, a.T, a.K, a.E, a.counts, a.offsets, a.meta, a.tiles_s, a.tiles_w, a.tiles_w2, a.row_token,
                   a.row_of, L.disp.bits, L.disp.d);
  }
  grid.sync();

  // gate/up + SwiGLU over the 16-row tiles, then the down projection
  gemm1_stream_run(bid, nb, L.g1, a.x, a.row_token, a.tiles_s, a.meta, a.w1, a.w3, a.ws1, a.ws3, a.h_routed,
                   a.h_shared, a.D, a.I, a.S, a.E);
  grid.sync();
  gemm2_stream_run<FD_THREADS / 64>(bid, nb, L.g2, a.h_routed, a.h_shared, a.tiles_s, a.meta, a.w2, a.ws2,
                                    a.o_routed, a.o_shared, nullptr, 1, a.T, a.D, a.I, a.S, a.E);
  grid.sync();

  // combine: a token per block
  for (int t = bid; t < a.T; t += nb) {
    combine_token<true, FD_THREADS>(t, 0, 1, L.comb.srow, L.comb.sw, a.idx, a.w, a.row_of, a.o_routed, a.o_shared,
                                    a.out, a.K, a.D);
    __syncthreads();
  }
}

bool decode_fused_ok(const Dims& d) {
  return d.dtype == 1 && d.T >= 1 && d.T <= kFusedMaxT && d.E <= kFusedMaxE && d.K <= kMaxTopK && d.G <= kMaxG;
}

hipError_t launch_decode_fused(const Dims& d, const ExpertPtrs& w, const void* w_gate, const float* bias,
                               float route_scale, bool softmax, const void* x, double* zpart, int nsplit, int32_t* idx,
                               float* wt, int32_t* counts, const Act& a, int32_t* row_of, void* out, hipStream_t s) {
  if (!decode_fused_ok(d) || nsplit > kMaxSplit) return hipErrorInvalidValue;
  const int nb = persistent_grid((const void*)decode_fused, FD_THREADS);
  FusedArgs f;
  f.x = static_cast<const bf16_t*>(x);
  f.w_gate = static_cast<const bf16_t*>(w_gate);
  f.bias = bias;
  f.w1 = static_cast<const bf16_t*>(w.w1);
  f.w3 = static_cast<const bf16_t*>(w.w3);
  f.w2 = static_cast<const bf16_t*>(w.w2);
  f.ws1 = static_cast<const bf16_t*>(w.ws1);
  f.ws3 = static_cast<const bf16_t*>(w.ws3);
  f.ws2 = static_cast<const bf16_t*>(w.ws2);
  f.zpart = zpart;
  f.idx = idx;
  f.counts = counts;
  f.offsets = const_cast<int32_t*>(a.offsets);
  f.row_token = const_cast<int32_t*>(a.row_token);
  f.row_of = row_of;
  f.meta = const_cast<int32_t*>(a.meta);
  f.w = wt;
  f.tiles_s = const_cast<Tile*>(a.tiles_skinny);
  f.tiles_w = const_cast<Tile*>(a.tiles_wide);
  f.tiles_w2 = const_cast<Tile*>(a.tiles_wide2);
  f.h_routed = static_cast<bf16_t*>(a.h_routed);
  f.h_shared = static_cast<bf16_t*>(a.h_shared);
  f.o_routed = static_cast<bf16_t*>(a.o_routed);
  f.o_shared = static_cast<bf16_t*>(a.o_shared);
  f.out = static_cast<bf16_t*>(out);
  f.T = (int)d.T;
  f.D = d.D;
  f.E = d.E;
  f.G = d.G;
  f.Gk = d.Gk;
  f.K = d.K;
  f.I = d.I;
  f.S = d.S;
  f.nsplit = nsplit;
  f.kslice = router_kslice(d, nsplit);
  f.softmax = softmax ? 1 : 0;
  f.route_scale = route_scale;
  void* args[] = {&f};
  Span sp("decode_fused", s);
  return hipLaunchCooperativeKernel((const void*)decode_fused, dim3(nb), dim3(FD_THREADS), args, 0, s);
}

}  // namespace moe

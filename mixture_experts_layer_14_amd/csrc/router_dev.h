// Device code of the router shared by its kernels and the fused decode kernel ("DeepSeek-V3.2-Exp ·
// Router", formula steps 1-4 and the Gate.forward excerpt).
#pragma once
#include <float.h>
#include <math.h>

#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Step 1: z = x W_r^T. Each 32-wide k chunk is one bf16 MFMA (products exact in
// fp32, chunk sum rounded once) and the chunks are summed in fp64, so z keeps
// well under 1e-7 absolute error before its single rounding to fp32. Partial
// sums over `nsplit` slices of D are written to zpart[split][T][E] (fp64) and
// added in slice order by router_select.
//
// Block: 4 waves on one tile of 32 tokens x 32 experts (2 x 2 MFMA tiles); wave w takes the
// w-th quarter of the block's slice (whole chunks) and wave 0 adds the four fp64 partial tiles
// in wave order. Grid (T/32, E/32, nsplit).
// ---------------------------------------------------------------------------
constexpr int kMaxSplit = 8;

// One tile (bx, by, split) on waves 0-3 of the calling block; waves 4 and up only take part in the
// block barrier. red: 3 x 16 x 64 doubles of LDS.
MOE_DEV void logits_tile(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg, double* __restrict__ zpart,
                         int T, int D, int E, int kslice, int bx, int by, int split, double (*red)[16][64]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave >= 4) {
    __syncthreads();
    return;
  }
  const int r = lane & 15, kq = lane >> 4;
  const int t0 = bx * 32;
  const int e0 = by * 32;
  const int sb = split * kslice;
  const int nch = max(0, min(D, sb + kslice) - sb) / 32;
  const int kb = sb + (nch * wave / 4) * 32;
  const int ke = sb + (nch * (wave + 1) / 4) * 32;

  const bf16_t* ap[2];
  bool av[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    int t = t0 + m * 16 + r;
    av[m] = t < T;
    ap[m] = x + (size_t)(av[m] ? t : 0) * D + kq * 8;
  }
  const bf16_t* bp[2];
  bool bv[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    int e = e0 + n * 16 + r;
    bv[n] = e < E;
    bp[n] = wg + (size_t)(bv[n] ? e : 0) * D + kq * 8;
  }
  double acc[2][2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][n][i] = 0.0;

  const i32x4 zero = {0, 0, 0, 0};
  const f32x4 fz = {0.f, 0.f, 0.f, 0.f};
  // U chunks per trip: all their loads are issued before the first MFMA (a wave's range is a
  // few dozen chunks at most, so without this each chunk would pay a full memory latency)
  constexpr int U = 4;
  auto chunk = [&](const i32x4 a[2], const i32x4 b[2]) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f32x4 p = mfma_bf16_16x16x32(a[m], b[n], fz);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][n][i] += (double)p[i];
      }
  };
  int k = kb;
  for (; k + 32 * U <= ke; k += 32 * U) {
    i32x4 a[U][2], b[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int m = 0; m < 2; ++m) a[u][m] = av[m] ? ld16(ap[m] + k + 32 * u) : zero;
#pragma unroll
      for (int n = 0; n < 2; ++n) b[u][n] = bv[n] ? ld16(bp[n] + k + 32 * u) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) chunk(a[u], b[u]);
  }
  for (; k < ke; k += 32) {
    i32x4 a[2], b[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) a[m] = av[m] ? ld16(ap[m] + k) : zero;
#pragma unroll
    for (int n = 0; n < 2; ++n) b[n] = bv[n] ? ld16(bp[n] + k) : zero;
    chunk(a, b);
  }

  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave - 1][m * 8 + n * 4 + i][lane] = acc[m][n][i];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][n][i] += red[w][m * 8 + n * 4 + i][lane];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      int e = e0 + n * 16 + r;
      if (e >= E) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int t = t0 + m * 16 + kq * 4 + i;
        if (t < T) zpart[((size_t)split * T + t) * E + e] = acc[m][n][i];
      }
    }
}

// ---------------------------------------------------------------------------
// Steps 2-4; TT threads per token (a whole 256-thread block for small batches, one wave
// otherwise); thread i of a token owns experts i, i + TT, ...
//   - z: the token's fp64 partial logits summed in slice order, rounded once to fp32
//   - s = sigmoid(z), or with softmax scoring s = exp(z - max z) / sum exp(z - max z) over the
//     token's experts (fp64, the sum taken per thread, then per wave in lane order, then over the
//     waves in order; rounded once to fp32); selection score sb = s + bias
//   - group score: best + second-best sb of the group (best alone without bias); groups of
//     2..64 experts (a power of two) sit on consecutive lanes and a butterfly finds them,
//     otherwise one thread per group scans it in LDS
//   - keep the Gk best groups (ties: lower group); experts of other groups drop to -inf
//   - choices in descending sb, ties to the lower index: with a block per token every expert
//     counts the masked scores ranked before it (rank k < K makes it choice k); with a wave per
//     token, K rounds of wave argmax
//   - weights: the chosen experts' s over their sum taken in choice order, times route_scale
//     (softmax scoring: the chosen s times route_scale, not renormalised)
// ---------------------------------------------------------------------------
constexpr int kMaxE = 1024, kMaxG = 64, kMaxK = 16;

// Reductions over the TT threads of one token: a wave (TT = 64) or the whole block (TT = 256,
// the wave results combined in wave order through sh[4]).
template <int TT>
MOE_DEV float token_max(float v, double* sh) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  if constexpr (TT == 64) {
    return v;
  } else {
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    const float r = fmaxf(fmaxf((float)sh[0], (float)sh[1]), fmaxf((float)sh[2], (float)sh[3]));
    __syncthreads();
    return r;
  }
}
template <int TT>
MOE_DEV double token_sum(double v, double* sh) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if constexpr (TT == 64) {
    return v;
  } else {
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    const double r = ((sh[0] + sh[1]) + sh[2]) + sh[3];
    __syncthreads();
    return r;
  }
}

// -inf for NaN (a group of +inf and -inf scores sums to NaN): ranks below every group score
MOE_DEV float nan_low(float v) { return __builtin_isnan(v) ? -INFINITY : v; }

MOE_DEV void top2_merge(float& b, float& c, float b2, float c2) {
  const float hi = fmaxf(b, b2), lo = fminf(b, b2);
  c = fmaxf(lo, fmaxf(c, c2));
  b = hi;
}

// LDS of one selection block: TPB token slots of TT * EPT experts each.
template <int EPT, int TPB, int TT>
struct SelectLds {
  __attribute__((aligned(16))) float s_all[TPB][TT * EPT];  // s
  __attribute__((aligned(16))) float m_all[TPB][TT * EPT];  // sb, then sb masked by kept groups
  float gsc_all[TPB][kMaxG];
  int keep_all[TPB][kMaxG];
  int sel_all[TPB][kMaxK];
  double red[4];  // block-wide reductions (one token per 256-thread block)
};

// Tokens bid * TPB .. bid * TPB + TPB - 1 on a block of NT threads: TT = NT / TPB threads per token,
// EPT experts per thread (E <= TT * EPT). Every thread of the block calls it.
template <int EPT, int TPB, int NT>
MOE_DEV void select_block(int bid, const double* __restrict__ zpart, int nsplit, const float* __restrict__ bias, int T,
                          int E, int G, int Gk, int K, float route_scale, int softmax, int32_t* __restrict__ idx_out,
                          float* __restrict__ w_out, SelectLds<EPT, TPB, NT / TPB>& L) {
#pragma clang fp contract(off)
  constexpr int TT = NT / TPB;
  static_assert(TT == 64 || TT == 256, "a wave or a 256-thread block per token");
  auto& s_all = L.s_all;
  auto& m_all = L.m_all;
  auto& gsc_all = L.gsc_all;
  auto& keep_all = L.keep_all;
  auto& sel_all = L.sel_all;
  double* red = L.red;
  const int tid = threadIdx.x % TT, slot = threadIdx.x / TT;
  const int t = min(bid * TPB + slot, T - 1);  // a block's spare slots redo the last token
  const bool writer = bid * TPB + slot < T;
  float* s_l = s_all[slot];
  float* m_l = m_all[slot];
  float* gsc = gsc_all[slot];
  int* keep = keep_all[slot];
  int* sel = sel_all[slot];
  const int gsize = E / G;
  const bool lanes_path = gsize >= 2 && gsize <= 64 && (gsize & (gsize - 1)) == 0;

  // all partial logits of this thread's experts requested at once
  const double* zt = zpart + (size_t)t * E;
  const size_t slice = (size_t)T * E;
  double part[EPT][kMaxSplit];
  float bb[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + TT * j;
#pragma unroll
    for (int p = 0; p < kMaxSplit; ++p) part[j][p] = (e < E && p < nsplit) ? zt[p * slice + e] : 0.0;
    bb[j] = (bias && e < E) ? bias[e] : 0.f;
  }
  float zf[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    double z = part[j][0];
#pragma unroll
    for (int p = 1; p < kMaxSplit; ++p)
      if (p < nsplit) z += part[j][p];
    zf[j] = (float)z;
  }
  float zmax = 0.f;
  double zsum = 1.0;
  if (softmax) {  // uniform: every thread of the token takes part in the reductions
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < EPT; ++j)
      if (tid + TT * j < E) mx = fmaxf(mx, zf[j]);
    zmax = token_max<TT>(mx, red);
    double sm = 0.0;
#pragma unroll
    for (int j = 0; j < EPT; ++j)
      if (tid + TT * j < E) sm += exp((double)zf[j] - (double)zmax);
    zsum = token_sum<TT>(sm, red);
  }
  float sbv[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + TT * j;
    const float sv = softmax ? (float)(exp((double)zf[j] - (double)zmax) / zsum)
                             : (float)(1.0 / (1.0 + exp(-(double)zf[j])));
    sbv[j] = bias ? sv + bb[j] : sv;
    // a NaN selection score (non-finite x or bias) ranks below every number, so the selection
    // below still yields K distinct experts in [0, E), equal scores in ascending index order
    if (__builtin_isnan(sbv[j])) sbv[j] = -INFINITY;
    if (e < E) {
      s_l[e] = sv;
      m_l[e] = sbv[j];
    } else {
      sbv[j] = -INFINITY;
    }
    if (lanes_path) {
      float b = sbv[j], c = -INFINITY;
      for (int off = gsize >> 1; off >= 1; off >>= 1) top2_merge(b, c, __shfl_xor(b, off), __shfl_xor(c, off));
      if (e < E && e % gsize == 0) gsc[e / gsize] = nan_low(bias ? b + c : b);
    }
  }
  __syncthreads();
  if (!lanes_path) {
    if (tid < G) {
      float b = -INFINITY, c = -INFINITY;
      const float* v = m_l + tid * gsize;
      for (int i = 0; i < gsize; ++i) top2_merge(b, c, v[i], -INFINITY);
      gsc[tid] = nan_low(bias ? b + c : b);
    }
    __syncthreads();
  }
  if (tid < G) {
    const float mine = gsc[tid];
    int rank = 0;
    for (int g = 0; g < G; ++g) {
      const float o = gsc[g];
      rank += (o > mine) || (o == mine && g < tid);
    }
    keep[tid] = (G == 1) || rank < Gk;
  }
  __syncthreads();
  float mv[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + TT * j;
    mv[j] = (e < E && keep[e / gsize]) ? sbv[j] : -INFINITY;
  }
  if constexpr (TT == 64) {
    // one wave per token: K rounds of wave argmax (ties: lower index)
    uint32_t taken = 0;
    for (int k = 0; k < K; ++k) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const int e = tid + TT * j;
        if (e < E && !((taken >> j) & 1u) && (mv[j] > bv || (mv[j] == bv && e < bi))) {
          bv = mv[j];
          bi = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (tid == 0) sel[k] = bi;
      if (bi % TT == tid) taken |= 1u << (bi / TT);
    }
  } else {
    // a block per token: each expert counts the masked scores ranked before it
    __syncthreads();  // every read of the unmasked m_l is done
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid + TT * j;
      if (e < E) m_l[e] = mv[j];
    }
    __syncthreads();
    int rank[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) rank[j] = 0;
    auto count = [&](float o, int e2) {
#pragma unroll
      for (int j = 0; j < EPT; ++j) rank[j] += (o > mv[j]) || (o == mv[j] && e2 < tid + TT * j);
    };
    const int E4 = E & ~3;
#pragma unroll 8  // several LDS reads in flight (they are broadcasts: one address per wave)
    for (int e4 = 0; e4 < E4; e4 += 4) {
      const float4 q = *reinterpret_cast<const float4*>(m_l + e4);
      count(q.x, e4);
      count(q.y, e4 + 1);
      count(q.z, e4 + 2);
      count(q.w, e4 + 3);
    }
    for (int e2 = E4; e2 < E; ++e2) count(m_l[e2], e2);
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid + TT * j;
      if (e < E && rank[j] < K) sel[rank[j]] = e;
    }
  }
  __syncthreads();
  if (writer && tid < K) {
    const int e = sel[tid];
    idx_out[(size_t)t * K + tid] = e;
    if (softmax) {
      w_out[(size_t)t * K + tid] = s_l[e] * route_scale;
    } else {
      float tot = s_l[sel[0]];
      for (int k = 1; k < K; ++k) tot = tot + s_l[sel[k]];
      w_out[(size_t)t * K + tid] = s_l[e] / tot * route_scale;
    }
  }
}

}  // namespace moe

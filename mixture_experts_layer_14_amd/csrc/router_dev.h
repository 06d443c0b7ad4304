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
//     token's experts (fp64, the sum taken per thread, then over the wave in a fixed tree of DPP
//     steps, then over the waves in order; rounded once to fp32); selection score sb = s + bias
//   - group score: best + second-best sb of the group (best alone without bias); groups of
//     2..64 experts (a power of two) sit on consecutive lanes and DPP steps find them,
//     otherwise one thread per group scans it in LDS
//   - keep the Gk best groups (ties: lower group); experts of other groups drop to -inf
//   - choices in descending sb, ties to the lower index: with a block per token every expert
//     counts the masked scores ranked before it (rank k < K makes it choice k); with a wave per
//     token, each lane sorts its own experts once and K rounds take the wave's best head (a DPP
//     max, then a ballot of the lanes holding it)
//   - weights: the chosen experts' s over their sum taken in choice order, times route_scale
//     (softmax scoring: the chosen s times route_scale, not renormalised)
// ---------------------------------------------------------------------------
constexpr int kMaxE = 1024, kMaxG = 64, kMaxK = 16;

// Cross-lane steps inside a wave through DPP: the value of another lane of the same row of 16
// (quad_perm, the mirrors) or of the row before (row_bcast), read by a VALU move. Lanes of rows
// outside ROWS keep `old`. Every lane of the wave must be active.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]: lane ^ 1
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]: lane ^ 2
constexpr int kDppMirror = 0x140;     // lane 15 - i of the row
constexpr int kDppHalfMirror = 0x141; // lane 7 - i of the half row
constexpr int kDppBcast15 = 0x142;    // lane 15 of the row before
constexpr int kDppBcast31 = 0x143;    // lane 31, to rows 2 and 3

template <int CTRL, int ROWS = 0xf>
MOE_DEV int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS = 0xf>
MOE_DEV float dpp_f(float old, float v) {
  return __int_as_float(dpp_i<CTRL, ROWS>(__float_as_int(old), __float_as_int(v)));
}

// Wave maximum (float) and minimum (int), returned to every lane: the row reduced with quad_perm
// and the mirrors, the rows joined with the broadcasts in lane 63, then read from there.
MOE_DEV float wave_max_f(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v, v));
  v = fmaxf(v, dpp_f<kDppXor2>(v, v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v, v));
  v = fmaxf(v, dpp_f<kDppMirror>(v, v));
  v = fmaxf(v, dpp_f<kDppBcast15, 0xa>(v, v));
  v = fmaxf(v, dpp_f<kDppBcast31, 0xc>(v, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Wave sum (fp64), returned to every lane: the same steps as the maximum, each adding the sums of
// two disjoint lane sets, so the additions form one fixed tree (lane pairs, quads, half rows, rows,
// row pairs) and the total does not depend on timing. Rows a broadcast skips add zero; only lane
// 63's value is read.
template <int CTRL, int ROWS = 0xf>
MOE_DEV double dpp_d(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = dpp_i<CTRL, ROWS>(0, (int)(b & 0xffffffffll));
  const int hi = dpp_i<CTRL, ROWS>(0, (int)(b >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
MOE_DEV double wave_sum_d(double v) {
  v = v + dpp_d<kDppXor1>(v);
  v = v + dpp_d<kDppXor2>(v);
  v = v + dpp_d<kDppHalfMirror>(v);
  v = v + dpp_d<kDppMirror>(v);
  v = v + dpp_d<kDppBcast15, 0xa>(v);
  v = v + dpp_d<kDppBcast31, 0xc>(v);
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), 63);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), 63);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
MOE_DEV int wave_min_i(int v) {
  v = min(v, dpp_i<kDppXor1>(v, v));
  v = min(v, dpp_i<kDppXor2>(v, v));
  v = min(v, dpp_i<kDppHalfMirror>(v, v));
  v = min(v, dpp_i<kDppMirror>(v, v));
  v = min(v, dpp_i<kDppBcast15, 0xa>(v, v));
  v = min(v, dpp_i<kDppBcast31, 0xc>(v, v));
  return __builtin_amdgcn_readlane(v, 63);
}

// Reductions over the TT threads of one token: a wave (TT = 64) or the whole block (TT = 256,
// the wave results combined in wave order through sh[4]).
template <int TT>
MOE_DEV float token_max(float v, double* sh) {
  v = wave_max_f(v);
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
  v = wave_sum_d(v);
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

// Best and second best (b, c) of each group of gsize consecutive lanes (a power of two, 2..64,
// groups aligned in the wave); the group's last lane ends with them. Each step joins two disjoint
// lane sets: lane pairs, quads, halves of a row (mirrors), rows (row 15 broadcast to the odd
// rows), row pairs (lane 31 to row 3). Lanes of rows a broadcast skips merge with -inf.
template <int CTRL, int ROWS = 0xf>
MOE_DEV void top2_step(float& b, float& c) {
  top2_merge(b, c, dpp_f<CTRL, ROWS>(-INFINITY, b), dpp_f<CTRL, ROWS>(-INFINITY, c));
}
MOE_DEV void group_top2(float& b, float& c, int gsize) {
  top2_step<kDppXor1>(b, c);
  if (gsize >= 4) top2_step<kDppXor2>(b, c);
  if (gsize >= 8) top2_step<kDppHalfMirror>(b, c);
  if (gsize >= 16) top2_step<kDppMirror>(b, c);
  if (gsize >= 32) top2_step<kDppBcast15, 0xa>(b, c);
  if (gsize >= 64) top2_step<kDppBcast31, 0xc>(b, c);
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
      group_top2(b, c, gsize);
      if (e < E && e % gsize == gsize - 1) gsc[e / gsize] = nan_low(bias ? b + c : b);
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
    // one wave per token. Each lane orders its experts by (masked score descending, index
    // ascending); experts past E hold -inf and the largest indices, so they come last and, with
    // K at most the experts of the kept groups, are never taken. Each round takes the wave's
    // best head: the DPP maximum of the heads, the lanes holding it by ballot (several only on
    // equal scores: then the lowest index of theirs), and the winning lane drops its head.
    float hv[EPT];
    int he[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      hv[j] = mv[j];
      he[j] = tid + TT * j;
    }
    // insertion sort, stable: the indices already ascend, so an equal score never moves up
#pragma unroll
    for (int j = 1; j < EPT; ++j)
#pragma unroll
      for (int i = j; i > 0; --i) {
        const bool up = hv[i] > hv[i - 1];
        const float v0 = hv[i - 1], v1 = hv[i];
        const int e0 = he[i - 1], e1 = he[i];
        hv[i - 1] = up ? v1 : v0;
        hv[i] = up ? v0 : v1;
        he[i - 1] = up ? e1 : e0;
        he[i] = up ? e0 : e1;
      }
    for (int k = 0; k < K; ++k) {
      const float best = wave_max_f(hv[0]);
      const unsigned long long hit = __ballot(hv[0] == best);
      const int win = __popcll(hit) == 1 ? __builtin_amdgcn_readlane(he[0], __builtin_ctzll(hit))
                                         : wave_min_i(hv[0] == best ? he[0] : 0x7fffffff);
      if (tid == 0) sel[k] = win;
      if (tid == win % TT) {
#pragma unroll
        for (int j = 0; j + 1 < EPT; ++j) {
          hv[j] = hv[j + 1];
          he[j] = he[j + 1];
        }
        hv[EPT - 1] = -INFINITY;
        he[EPT - 1] = 0x7fffffff;
      }
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

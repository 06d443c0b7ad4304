"""CPU oracle of the DeepSeek-V3-style MoE block forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, links or runs
this file: only the tests, the smoke check and the bench's cpu_baseline leg
do. It shares no code with the HIP kernels and imports nothing from them.

Plain, slow, obviously-correct numpy in float64, written from three pages:
  * "DeepSeek-V3.2-Exp · Router" (atlas.klimoza.dev, router inspector): the four
    formula steps z = x W_r, s = sigma(z), E_sel = top-8 of (s + b) within the top
    4 groups, G_i = 2.5 s_i E_i / sum_j s_j E_j; and the Gate.forward excerpt
    (group view, top-2-sum group score, group mask, expert top-k, gather of the
    unbiased scores, renormalisation, route scale).
  * "DeepSeek-V3.2-Exp · Mixture of experts" (open-model-atlas, MoE block):
    the block's output, a per-token sum of the routed experts' outputs weighted
    by the gate plus the shared expert's output, accumulated in fp32 in expert
    order with the shared expert last (MoE.forward excerpt); the per-expert token
    lists in token order (dispatch); the parameter table (three 7168x2048
    matrices per expert).

  * "Hardware for DeepSeek-V3 and R1: Why a 671B MoE Model Needs So Much
    Memory", section "Why the dense layers and shared expert matter": the first
    three layers are ordinary dense feed-forward blocks with an intermediate
    size of 18,432 (dense_ffn).

Readings where the pages are silent (numbered as in the design notes, where R10-R12 and
R14 concern the ABI and the test rules):
  R1  the linear of the router has no bias; its dot product is exact (fp64
      sum of exact bf16 / fp32 products) and rounded once to fp32.
  R2  sigmoid evaluated in fp64, rounded once to fp32.
  R3  the selection bias is an explicit input, used in every workload.
  R4  ties in every top-k go to the lower index; top-k output is in
      descending order (the excerpt's topk is sorted).
  R5  the renormalising sum runs in rank order, in fp32.
  R6  the expert is the 3-matrix SwiGLU  w2( silu(w1 x) * (w3 x) ), no biases
      (the count 3 * 7168 * 2048 per expert leaves no room for biases).
  R7  the SwiGLU activation h is formed in fp32 and stored in the activation
      dtype (fp32; bf16; or e4m3 with one fp32 scale per token per 128 columns);
      each expert's output row is rounded to x's dtype before the weighted add.
  R8  combine order is the excerpt's loop order: routed experts ascending, then
      the shared expert; every add and multiply rounds to fp32; the result is
      cast to x's dtype.
  R9  FP8 (OCP e4m3fn, bias 7, max 448, no infinities): scale = amax / 448
      (1 when amax = 0), code = round-to-nearest-even(v / scale), saturating.
  R13 softmax scoring (the excerpt's other branch): exp(z - max z) over the
      token's experts divided by their sum, in fp64, rounded once to fp32; the
      gathered softmax scores are not renormalised (the excerpt renormalises
      only the sigmoid branch) before the route scale.
  R15 the dense feed-forward is the MLP the MoE block page uses for its shared
      expert (same R6 form, same R7 roundings), applied to every token; no
      router, no weighting, its output row is the result.

Functions and their pins (tests/test_oracle_*.py):
  bf16 / e4m3 codecs      torch's bfloat16 / float8_e4m3fn casts; spec values
  quant_1x128             amax maps to code 448; zero block; RNE error bound;
                          a hand-worked 1x128 row (exact codes, both tie cases,
                          the smallest subnormal)
  store_act("fp8")        torch's float8_e4m3fn cast of h / (amax / 448) per
                          token per 128 columns, bit for bit, on a SwiGLU h
                          written with torch.nn.functional; per-token scales
                          (two tokens of different amax in one column block)
  router_logits           exact rational dot product (fractions) on tiny inputs;
                          identity router weight gives z = x
  sigmoid32               scipy.special.expit; sigma(0) = 0.5
  softmax scoring         scipy.special.softmax; weights are the gathered
                          scores times the scale; shift invariance; no-bias
                          single group = top-k of z; group-max brute force
  route                   brute-force enumeration of group and expert subsets;
                          hand-worked group-score case; invariants (8 distinct,
                          <= 4 groups, sum 2.5); bias-shift invariance;
                          special cases G=1 / b=0 / E=K
  dispatch                lexsort of (expert, token) keys; permutation invariants
  swiglu_rows             torch.nn.functional silu / linear in fp64 (f32, bf16,
                          and fp8 with torch's float8 requantisation of h)
  moe_forward             dense-G formulation bit-exact; x=0; W2 doubling;
                          token-permutation equivariance; E=K=1 reduces to
                          2.5 * MLP + shared MLP
  dense_ffn               equals the block with one expert, K = 1, scale 1 and
                          a zero shared down projection, bit for bit;
                          torch.nn.functional MLP; 1x1 closed form (silu on the
                          W1 branch); x = 0; W2 doubling; token permutation
Full-shape output values have no printed example on the pages: beyond the
pins above they are parity unpinned.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional, Tuple

import numpy as np

f32 = np.float32
f64 = np.float64

# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(f32)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(v, dtype=f32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16, returned as exact float32 values."""
    return bf16_bits_to_f32(f32_to_bf16_bits(v))


E4M3_MAX = 448.0


def _e4m3_table() -> np.ndarray:
    """Value of each non-negative e4m3fn code 0..126 (127 is NaN)."""
    vals = np.empty(127, dtype=f64)
    for code in range(127):
        e, m = code >> 3, code & 7
        vals[code] = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_POS = _e4m3_table()


def _e4m3_all() -> np.ndarray:
    """Value of every e4m3fn code 0..255: the sign bit over the magnitude table; S.1111.111 is NaN."""
    mag = np.concatenate([_E4M3_POS, [np.nan]])
    return np.concatenate([mag, -mag])


_E4M3_ALL = _e4m3_all()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3fn codes (uint8) -> float64 values (NaN for S.1111.111), by table lookup."""
    return _E4M3_ALL[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float values -> e4m3fn codes: round to nearest, ties to the even code, saturate at 448.
    The sign of zero is kept."""
    v = np.asarray(v, dtype=f64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")  # first table value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(_E4M3_POS[hi] == a, hi, code)
    sign = np.signbit(v).astype(np.uint8) << 7
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quant_1x128(a: np.ndarray, block: int = 128) -> Tuple[np.ndarray, np.ndarray]:
    """Per row, per `block` consecutive columns: scale = fp32(amax / 448) (1 if amax == 0),
    code = e4m3(fp32(a / scale)). a is float32 [n, C] with C % block == 0."""
    a = np.asarray(a, dtype=f32)
    n, c = a.shape
    blk = a.reshape(n, c // block, block)
    amax = np.abs(blk).max(axis=2)
    scale = np.where(amax > 0, (amax / f32(E4M3_MAX)).astype(f32), f32(1.0)).astype(f32)
    q = (blk / scale[:, :, None]).astype(f32)
    return e4m3_encode(q).reshape(n, c), scale


def dequant_1x128(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    n, c = codes.shape
    v = e4m3_decode(codes).reshape(n, c // block, block) * scales.astype(f64)[:, :, None]
    return v.reshape(n, c)


def dequant_128x128(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """e4m3 weight [R, C] with one scale per block x block tile -> float64 values."""
    r, c = codes.shape
    v = e4m3_decode(codes)
    v.reshape(r // block, block, c // block, block)[...] *= scales.astype(f64)[:, None, :, None]
    return v


# --------------------------------------------------------------------------
# Router (router page: steps 1-4 and Gate.forward)
# --------------------------------------------------------------------------


def router_logits(x: np.ndarray, w_gate: np.ndarray) -> np.ndarray:
    """Step 1, z = x W_r: fp64 dot products of the exact inputs, rounded once to fp32 (R1).
    x [T, D], w_gate [E, D] (router weight stored [experts, dim])."""
    return (np.asarray(x, f64) @ np.asarray(w_gate, f64).T).astype(f32)


def sigmoid32(z: np.ndarray) -> np.ndarray:
    """Step 2, s = sigma(z), evaluated in fp64 and rounded once to fp32 (R2)."""
    z = np.asarray(z, f64)
    with np.errstate(over="ignore"):
        return (1.0 / (1.0 + np.exp(-z))).astype(f32)


def _topk_desc(values: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries of each row, descending, ties to the lower index (R4)."""
    order = np.argsort(-values, axis=-1, kind="stable")
    return order[..., :k]


@dataclass
class Route:
    idx: np.ndarray        # int32 [T, K], descending biased score
    w: np.ndarray          # fp32 [T, K], aligned with idx
    s: np.ndarray          # fp32 [T, E] unbiased scores
    sb: np.ndarray         # fp32 [T, E] selection scores (s + b)
    masked: np.ndarray     # fp32 [T, E] selection scores with non-kept groups at -inf
    group_scores: Optional[np.ndarray]  # fp32 [T, G]
    kept_groups: Optional[np.ndarray]   # int [T, Gk]


def route_from_logits(cfg, z: np.ndarray, bias: Optional[np.ndarray],
                      score_func: Optional[str] = None) -> Route:
    """Steps 2-4 on fp32 logits z [T, E]. score_func: "sigmoid" or "softmax" (the excerpt's two
    branches); None takes cfg.score_func, else sigmoid."""
    if score_func is None:
        score_func = getattr(cfg, "score_func", "sigmoid")
    z = np.asarray(z, f32)
    t, e = z.shape
    g, gk, k = cfg.n_groups, cfg.topk_groups, cfg.topk
    if score_func == "softmax":
        zz = z.astype(f64)
        ez = np.exp(zz - zz.max(axis=1, keepdims=True))
        s = (ez / ez.sum(axis=1, keepdims=True)).astype(f32)
    else:
        s = sigmoid32(z)
    sb = (s + np.asarray(bias, f32)).astype(f32) if bias is not None else s.copy()
    gs = kept = None
    masked = sb.copy()
    if g > 1:
        grouped = sb.reshape(t, g, e // g)  # group j holds experts j*E/G .. (j+1)*E/G - 1
        if bias is None:
            gs = grouped.max(axis=2)
        else:
            top2 = -np.sort(-grouped, axis=2)[:, :, :2]
            gs = (top2[:, :, 0] + top2[:, :, 1]).astype(f32)
        kept = _topk_desc(gs, gk)
        keep = np.zeros((t, g), dtype=bool)
        np.put_along_axis(keep, kept, True, axis=1)
        masked = np.where(np.repeat(keep, e // g, axis=1), sb, f32(-np.inf)).astype(f32)
    idx = _topk_desc(masked, k).astype(np.int32)
    w = np.take_along_axis(s, idx, axis=1).astype(f32)
    if score_func == "sigmoid":
        tot = w[:, 0].copy()
        for j in range(1, k):          # R5: rank-order fp32 sum
            tot = (tot + w[:, j]).astype(f32)
        w = (w / tot[:, None]).astype(f32)
    w = (w * f32(cfg.route_scale)).astype(f32)
    return Route(idx, w, s, sb, masked, gs, kept)


def route(cfg, x: np.ndarray, w_gate: np.ndarray, bias: Optional[np.ndarray],
          score_func: Optional[str] = None) -> Route:
    """The router: (weights [T, K] fp32, indices [T, K]) for tokens x [T, D]."""
    return route_from_logits(cfg, router_logits(x, w_gate), bias, score_func)


def dense_gate(r: Route, n_experts: int) -> np.ndarray:
    """G [T, E]: the K weights spread over all experts, zero elsewhere (router page, G_i)."""
    gmat = np.zeros((r.idx.shape[0], n_experts), dtype=f32)
    np.put_along_axis(gmat, r.idx.astype(np.int64), r.w, axis=1)
    return gmat


@dataclass
class NearTies:
    group: np.ndarray     # bool [T]: kept/dropped group boundary gap < thresh
    boundary: np.ndarray  # bool [T]: K-th vs (K+1)-th expert gap < thresh
    order: np.ndarray     # bool [T]: adjacent pair among the K chosen closer than thresh

    @property
    def any(self) -> np.ndarray:
        return self.group | self.boundary | self.order


def near_ties(cfg, r: Route, thresh: float = 1e-6) -> NearTies:
    """Flag tokens whose selection could flip under a perturbation below `thresh`."""
    t = r.idx.shape[0]
    k = cfg.topk
    grp = np.zeros(t, dtype=bool)
    if r.group_scores is not None and cfg.topk_groups < cfg.n_groups:
        gsort = -np.sort(-r.group_scores.astype(f64), axis=1)
        grp = (gsort[:, cfg.topk_groups - 1] - gsort[:, cfg.topk_groups]) < thresh
    msort = -np.sort(-r.masked.astype(f64), axis=1)
    bnd = np.zeros(t, dtype=bool)
    if k < msort.shape[1]:
        nxt = msort[:, k]
        bnd = np.isfinite(nxt) & ((msort[:, k - 1] - nxt) < thresh)
    ordr = np.zeros(t, dtype=bool)
    if k > 1:
        ordr = (np.diff(-msort[:, :k], axis=1) < thresh).any(axis=1)
    return NearTies(grp, bnd, ordr)


# --------------------------------------------------------------------------
# Dispatch (MoE block page: bincount, per-expert torch.where in token order)
# --------------------------------------------------------------------------


def dispatch(idx: np.ndarray, n_experts: int):
    """counts [E], offsets [E+1] (exclusive scan), row_token [T*K] (rows grouped by expert
    ascending, tokens ascending inside an expert), row_of [T, K] (row of each assignment)."""
    idx = np.asarray(idx)
    t, k = idx.shape
    counts = np.zeros(n_experts, dtype=np.int64)
    for tok in range(t):
        for j in range(k):
            counts[idx[tok, j]] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:-1].copy()
    row_token = np.empty(t * k, dtype=np.int64)
    row_of = np.empty((t, k), dtype=np.int64)
    for tok in range(t):            # tokens in ascending order -> stable inside each expert
        for j in range(k):
            e = idx[tok, j]
            row = fill[e]
            fill[e] += 1
            row_token[row] = tok
            row_of[tok, j] = row
    return (counts.astype(np.int32), offsets.astype(np.int32),
            row_token.astype(np.int32), row_of.astype(np.int32))


# --------------------------------------------------------------------------
# Experts (R6, R7)
# --------------------------------------------------------------------------


def store_act(h: np.ndarray, act: str) -> np.ndarray:
    """h (fp64) -> value seen by the down projection (fp64), per R7."""
    h32 = np.asarray(h, f64).astype(f32)
    if act == "f32":
        return h32.astype(f64)
    if act == "bf16":
        return round_bf16(h32).astype(f64)
    if act == "fp8":
        q, sc = quant_1x128(h32)
        return dequant_1x128(q, sc)
    raise ValueError(act)


def round_out(o: np.ndarray, out_dtype: str) -> np.ndarray:
    """Expert output row -> x's dtype, returned as fp32 values."""
    o32 = np.asarray(o, f64).astype(f32)
    return o32 if out_dtype == "f32" else round_bf16(o32)


def swiglu_rows(xr: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray,
                act: str, out_dtype: str) -> np.ndarray:
    """Rows xr [n, D] through w2( silu(w1 x) * (w3 x) ); w1, w3 [I, D], w2 [D, I] ([out, in]).
    Returns the rows in x's dtype as fp32 values."""
    xr = np.asarray(xr, f64)
    g = xr @ np.asarray(w1, f64).T
    u = xr @ np.asarray(w3, f64).T
    with np.errstate(over="ignore"):
        h = g / (1.0 + np.exp(-g)) * u
    hs = store_act(h, act)
    o = hs @ np.asarray(w2, f64).T
    return round_out(o, out_dtype)


# --------------------------------------------------------------------------
# The block (MoE block page: MoE.forward)
# --------------------------------------------------------------------------

ExpertFn = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]


def activation_input(x: np.ndarray, act: str) -> np.ndarray:
    """What the expert GEMMs read for x: x itself, or its per-token 1x128 e4m3 image (R9)."""
    x = np.asarray(x, f64)
    if act != "fp8":
        return x
    q, sc = quant_1x128(x.astype(f32))
    return dequant_1x128(q, sc)


@dataclass
class Forward:
    out: np.ndarray      # fp32 values of the output in x's dtype [T, D]
    route: Route
    dispatch: tuple


def moe_forward(cfg, x: np.ndarray, w_gate: np.ndarray, bias: Optional[np.ndarray],
                expert: ExpertFn, shared: Callable[[], Tuple[np.ndarray, np.ndarray, np.ndarray]],
                act: str, out_dtype: str) -> Forward:
    """Delta [T, D] for tokens x [T, D] (exact input values).

    The block's defining sum (router page, G_i; MoE block page, block output): per token,
    Delta = sum over experts e ascending of G_e * FFN_e(x) + FFN_shared(x), where G_e is the
    token's routing weight for e and zero for the experts it did not choose. A zero term adds an
    exact zero to the fp32 accumulator, so only each expert's chosen tokens are evaluated: an
    expert no token chose is never read. The dispatch permutation is computed on its own and
    returned for the tests; the sum does not use it.

    expert(e) -> (w1, w3, w2) fp64 of routed expert e; shared() -> the shared expert's.
    act: activation storage dtype ("f32" | "bf16" | "fp8"); out_dtype: x's dtype."""
    x = np.asarray(x, f64)
    t, d = x.shape
    r = route(cfg, x, w_gate, bias)
    gate = dense_gate(r, cfg.n_experts)                # G [T, E]
    chosen = np.zeros((t, cfg.n_experts), dtype=bool)
    np.put_along_axis(chosen, r.idx.astype(np.int64), True, axis=1)
    xa = activation_input(x, act)
    y = np.zeros((t, d), dtype=f32)
    for e in range(cfg.n_experts):                     # R8: ascending expert order
        toks = np.nonzero(chosen[:, e])[0]
        if toks.size == 0:
            continue
        w1, w3, w2 = expert(e)
        o = swiglu_rows(xa[toks], w1, w3, w2, act, out_dtype)
        y[toks] = (y[toks] + (o * gate[toks, e][:, None]).astype(f32)).astype(f32)
    w1, w3, w2 = shared()
    y = (y + swiglu_rows(xa, w1, w3, w2, act, out_dtype)).astype(f32)
    out = y if out_dtype == "f32" else round_bf16(y)
    return Forward(out, r, dispatch(r.idx, cfg.n_experts))


def moe_forward_dense(cfg, x: np.ndarray, w_gate: np.ndarray, bias: Optional[np.ndarray],
                      expert: ExpertFn, shared, act: str, out_dtype: str) -> np.ndarray:
    """The same Delta written with the dense gate G of the router page: every expert runs on every
    token and is weighted by G (zero for the 248 unselected), summed over experts ascending.
    Only for tiny shapes."""
    x = np.asarray(x, f64)
    r = route(cfg, x, w_gate, bias)
    gmat = dense_gate(r, cfg.n_experts)
    xa = activation_input(x, act)
    y = np.zeros(x.shape, dtype=f32)
    for e in range(cfg.n_experts):
        w1, w3, w2 = expert(e)
        o = swiglu_rows(xa, w1, w3, w2, act, out_dtype)
        y = (y + (o * gmat[:, e:e + 1]).astype(f32)).astype(f32)
    w1, w3, w2 = shared()
    y = (y + swiglu_rows(xa, w1, w3, w2, act, out_dtype)).astype(f32)
    return y if out_dtype == "f32" else round_bf16(y)


def dense_ffn(x: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray, act: str,
              out_dtype: str) -> np.ndarray:
    """The first layers' dense feed-forward (R15) on tokens x [T, D] (exact input values): the
    image of x the GEMMs read (R9 for fp8), then w2( silu(w1 x) * (w3 x) ) with the R7 roundings.
    w1, w3 [I, D], w2 [D, I] fp64 ([out, in]). Returns the rows in x's dtype as fp32 values."""
    return swiglu_rows(activation_input(x, act), w1, w3, w2, act, out_dtype)


def param_count(dim: int, n_experts: int, inter: int, n_shared: int, bias: bool = True) -> dict:
    """Learned parameters of one block, counted from the tensor shapes the oracle consumes."""
    router = n_experts * dim + (n_experts if bias else 0)
    expert = 3 * dim * inter
    return dict(router=router, expert=expert, shared=3 * dim * inter * n_shared,
                block=router + n_experts * expert + 3 * dim * inter * n_shared)


def flops_per_token(dim: int, n_experts: int, topk: int, inter: int, n_shared: int) -> int:
    """Multiply-adds x2 per token: router GEMV plus K routed and the shared SwiGLU experts."""
    return 2 * dim * n_experts + 2 * 3 * dim * inter * (topk + n_shared)


"""Parity rules between the HIP path and the oracle (used by the GPU tests and the bench).

Routing: expert indices must equal the oracle's, order included; a token may differ only if the
oracle flags it as a near-tie (a score gap below 1e-6 at the kept-group boundary, the K-th expert
boundary, or between two chosen experts), and at most 0.01% of the tokens may differ.
Weights: within 4 ulp of the oracle's where the indices agree.
A token that differs must still be a valid group-limited top-k of the oracle's fp32 scores when
every gap below 1e-6 may be resolved either way.
Dispatch: counts, offsets, row_token and row_of equal the oracle's dispatch of the GPU's indices.
Outputs: relative L2 error (fp64) at most 1e-4 (fp32 blocks), 1e-2 (bf16), 5e-2 (fp8), both over
all compared values and for every compared token on its own.
"""
import math
import sys

import numpy as np
import torch

from oracle import moe_oracle as O

REL_L2 = {"f32": 1e-4, "bf16": 1e-2, "fp8": 5e-2}
NEAR_TIE = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np_i32(t):
    return t.detach().to("cpu").numpy().astype(np.int64)


def valid_selection(shape, r, t, sel, thresh=NEAR_TIE):
    """Is `sel` (the K experts a kernel chose for token t, in its order) a valid group-limited
    top-k of the oracle's fp32 scores of token t, if every gap below `thresh` may go either way?
    The kept groups must be the touched ones plus the best others; each touched group within
    thresh of the Gk-th group score; each chosen expert within thresh of the K-th best score of
    the kept groups; the order descending within thresh."""
    E, G, Gk, K = shape.n_experts, shape.n_groups, shape.topk_groups, shape.topk
    sel = np.asarray(sel, dtype=np.int64)
    if len(set(sel.tolist())) != K or sel.min() < 0 or sel.max() >= E:
        return False
    sb = r.sb[t].astype(np.float64)
    gsize = E // G
    kept = np.ones(G, dtype=bool)
    if G > 1 and r.group_scores is not None and Gk < G:
        gs = r.group_scores[t].astype(np.float64)
        touched = np.unique(sel // gsize)
        if len(touched) > Gk:
            return False
        gk_th = np.sort(gs)[::-1][Gk - 1]
        if (gs[touched] < gk_th - thresh).any():
            return False
        kept = np.zeros(G, dtype=bool)
        kept[touched] = True
        for g in np.argsort(-gs, kind="stable"):
            if kept.sum() >= Gk:
                break
            kept[g] = True
    cand = np.where(np.repeat(kept, gsize), sb, -np.inf)
    kth = np.sort(cand)[::-1][K - 1]
    if (cand[sel] < kth - thresh).any():
        return False
    return bool((np.diff(sb[sel]) <= thresh).all())


def route_check(shape, oracle_route, gpu_idx, gpu_w):
    """Returns (mismatched token mask, report dict); asserts the routing rules."""
    oi = oracle_route.idx.astype(np.int64)
    gi = np.asarray(gpu_idx).astype(np.int64)
    assert gi.shape == oi.shape
    bad = (gi != oi).any(axis=1)
    flags = O.near_ties(shape, oracle_route, NEAR_TIE)
    n = oi.shape[0]
    rep = dict(tokens=n, mismatched=int(bad.sum()), flagged=int(flags.any.sum()),
               flagged_group=int(flags.group.sum()), flagged_boundary=int(flags.boundary.sum()),
               flagged_order=int(flags.order.sum()))
    assert not (bad & ~flags.any).any(), f"unflagged routing mismatch: {rep}"
    assert bad.sum() <= math.floor(1e-4 * n), f"too many near-tie mismatches: {rep}"
    for t in np.nonzero(bad)[0]:
        assert valid_selection(shape, oracle_route, t, gi[t]), f"token {t}: {gi[t]} is no valid top-k: {rep}"
    ow = oracle_route.w
    gw = np.asarray(gpu_w, dtype=np.float32)
    ok = ~bad
    ulp = np.abs(gw[ok].view(np.int32).astype(np.int64) - ow[ok].view(np.int32).astype(np.int64))
    rep["w_max_ulp"] = int(ulp.max()) if ulp.size else 0
    if getattr(shape, "score_func", "sigmoid") == "softmax":
        # A softmax weight depends on every logit of its token: with logit errors |dz| (the
        # kernel's 32-product chunks are rounded to fp32 before their fp64 sum, <= ~1e-6 at
        # these sizes, plus the final rounding) its relative error is at most
        # |dz_e| + sum_j s_j |dz_j| <= 2 max |dz|; allowed: 4e-6.
        rel = np.abs(gw[ok].astype(np.float64) - ow[ok]) / np.abs(ow[ok].astype(np.float64))
        rep["w_max_rel"] = float(rel.max()) if rel.size else 0.0
        assert rep["w_max_rel"] <= 4e-6, rep
    else:
        # a sigmoid weight depends on its own logit and the K chosen scores: <= 4 ulp
        assert rep["w_max_ulp"] <= 4, rep
    return bad, rep


def dispatch_check(shape, gpu_idx, counts, offsets, row_token, row_of):
    c, o, rt, ro = O.dispatch(np.asarray(gpu_idx), shape.n_experts)
    assert np.array_equal(np.asarray(counts), c)
    assert np.array_equal(np.asarray(offsets), o)
    assert np.array_equal(np.asarray(row_token), rt)
    assert np.array_equal(np.asarray(row_of).reshape(ro.shape), ro)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a))


def out_check(shape, gpu_out, oracle_out, skip=None):
    g = np.asarray(gpu_out, np.float64)
    o = np.asarray(oracle_out, np.float64)
    if skip is not None and skip.any():
        g, o = g[~skip], o[~skip]
    err = rel_l2(g, o)
    per_tok = np.array([rel_l2(g[i], o[i]) for i in range(g.shape[0])])
    tol = REL_L2[shape.dtype]
    worst = int(per_tok.argmax()) if per_tok.size else -1
    rep = dict(rel_l2=err, max_token_rel_l2=float(per_tok.max()) if per_tok.size else 0.0, tol=tol,
               tokens=int(g.shape[0]))
    assert np.isfinite(g).all()
    assert err <= tol, rep
    assert (per_tok <= tol).all(), dict(rep, worst_token=worst, over=int((per_tok > tol).sum()))
    return rep


def tile_tokens(T, counts, offsets, row_token, bm, rng, per_expert="all", shared_stride=1):
    """Tokens such that the compared outputs hold at least one row of every `bm`-row M-tile the
    GEMM kernels ran: per routed expert every M-tile (per_expert="all") or its first, a middle
    and its last one ("ends"), each M-tile's row drawn at random except the last (ragged) tile's,
    which is its last row; then every `shared_stride`-th M-tile of the shared expert (tokens
    j*bm .. j*bm+bm-1) and the last token."""
    counts = np.asarray(counts)
    offsets = np.asarray(offsets)
    row_token = np.asarray(row_token)
    toks = [T - 1]
    for e in np.nonzero(counts)[0]:
        c = int(counts[e])
        mt = (c + bm - 1) // bm
        tiles = range(mt) if per_expert == "all" else sorted({0, mt // 2, mt - 1})
        for m in tiles:
            last = min(c, (m + 1) * bm) - 1
            row = last if m == mt - 1 else m * bm + int(rng.integers(0, bm))
            toks.append(int(row_token[offsets[e] + row]))
    for j in range(0, (T + bm - 1) // bm, shared_stride):
        toks.append(min(T - 1, j * bm + int(rng.integers(0, bm))))
    return np.unique(np.asarray(toks, dtype=np.int64))


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float32).numpy()

"""Parity rules between the HIP path and the oracle (used by the GPU tests and the bench).

Routing: expert indices must equal the oracle's, order included; a token may differ only if the
oracle flags it as a near-tie (a score gap below 1e-6 at the kept-group boundary, the K-th expert
boundary, or between two chosen experts), and at most 0.01% of the tokens may differ.
Weights: within 4 ulp of the oracle's where the indices agree.
Dispatch: counts, offsets, row_token and row_of equal the oracle's dispatch of the GPU's indices.
Outputs: relative L2 error (fp64) at most 1e-4 (fp32 blocks), 1e-2 (bf16), 5e-2 (fp8).
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
    per_tok = [rel_l2(g[i], o[i]) for i in range(g.shape[0])]
    rep = dict(rel_l2=err, max_token_rel_l2=max(per_tok) if per_tok else 0.0, tol=REL_L2[shape.dtype])
    assert np.isfinite(g).all()
    assert err <= REL_L2[shape.dtype], rep
    return rep


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float32).numpy()

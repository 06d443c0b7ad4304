"""Pins of the oracle's router (router page: steps 1-4, Gate.forward) and dispatch
(MoE block page: bincount and per-expert token gather)."""
import itertools
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import pytest
import scipy.special

from oracle import moe_oracle as O


def cfg(E=16, G=4, Gk=2, K=4, scale=2.5):
    return SimpleNamespace(n_experts=E, n_groups=G, topk_groups=Gk, topk=K, route_scale=scale)


def round_f32_exact(fr: Fraction) -> np.float32:
    """Correctly rounded fp32 of an exact rational (ties to even), by checking neighbours."""
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - fr),
                                     int(np.float32(v).view(np.uint32)) & 1))
    return np.float32(best)


def test_logits_correctly_rounded_vs_exact_rationals():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((6, 37)).astype(np.float32)
    w = (rng.standard_normal((5, 37)) * 0.3).astype(np.float32)
    z = O.router_logits(x, w)
    assert z.dtype == np.float32
    for t in range(6):
        for e in range(5):
            exact = sum(Fraction(float(x[t, d])) * Fraction(float(w[e, d])) for d in range(37))
            assert z[t, e] == round_f32_exact(exact)


def test_logits_identity_weight():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((9, 16)).astype(np.float32)
    assert np.array_equal(O.router_logits(x, np.eye(16, dtype=np.float32)), x)


def test_sigmoid_matches_expit():
    rng = np.random.default_rng(12)
    z = (rng.standard_normal(50_000) * 4).astype(np.float32)
    ours = O.sigmoid32(z)
    ref = scipy.special.expit(z.astype(np.float64)).astype(np.float32)
    ulps = np.abs(ours.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1 and (ulps > 0).sum() <= 5
    assert O.sigmoid32(np.float32([0.0]))[0] == 0.5


def test_group_score_is_sum_of_top2_not_max():
    """Hand-worked: 8 experts in 4 groups of 2, keep 2 groups, pick 2 experts, no bias offset.
    Group 0 = (3, -5): biggest single score but sum sigma(3)+sigma(-5) = 0.959;
    group 1 = (1, 1): sum 1.462; group 2 = (0.5, 0.4): 1.221; group 3 = (-1, -1): 0.538.
    Top-2-sum keeps groups {1, 2}; the two best experts there are 2 and 3 (equal scores, lower index
    first), each weighted 2.5 * s / (2 s) = 1.25 exactly. A max-based group score would keep {0, 1}
    and pick expert 0."""
    c = cfg(E=8, G=4, Gk=2, K=2)
    z = np.float32([[3.0, -5.0, 1.0, 1.0, 0.5, 0.4, -1.0, -1.0]])
    r = O.route_from_logits(c, z, np.zeros(8, np.float32))
    assert sorted(r.kept_groups[0].tolist()) == [1, 2]
    assert r.idx[0].tolist() == [2, 3]
    assert r.w[0].tolist() == [1.25, 1.25]
    # without a bias the excerpt scores a group by its maximum instead
    r2 = O.route_from_logits(c, z, None)
    assert sorted(r2.kept_groups[0].tolist()) == [0, 1] and r2.idx[0].tolist() == [0, 2]


def test_bias_selects_but_does_not_weight():
    """All logits 0 (s = 0.5). A +10 bias on expert 2 makes it first; the next is the lowest-index
    tie. The weights come from the unbiased scores: 2.5 * 0.5 / 1.0 = 1.25 each."""
    c = cfg(E=4, G=1, Gk=1, K=2)
    r = O.route_from_logits(c, np.zeros((1, 4), np.float32), np.float32([0, 0, 10, 0]))
    assert r.idx[0].tolist() == [2, 0]
    assert r.w[0].tolist() == [1.25, 1.25]


def _brute_route(c, sb):
    """Enumerate every kept-group subset and every expert subset (tiny shapes only)."""
    E, G, Gk, K = c.n_experts, c.n_groups, c.topk_groups, c.topk
    gsz = E // G
    gs = []
    for g in range(G):
        vals = [sb[g * gsz + i] for i in range(gsz)]
        gs.append(max(np.float32(vals[i] + vals[j]) for i in range(gsz) for j in range(gsz) if i != j))
    best_groups = max(itertools.combinations(range(G), Gk), key=lambda S: sum(float(gs[g]) for g in S))
    allowed = [e for g in best_groups for e in range(g * gsz, (g + 1) * gsz)]
    best_experts = max(itertools.combinations(allowed, K), key=lambda S: sum(float(sb[e]) for e in S))
    return gs, set(best_groups), set(best_experts)


def test_brute_force_enumeration_tiny():
    rng = np.random.default_rng(13)
    c = cfg(E=16, G=4, Gk=2, K=4)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    wg = (rng.standard_normal((16, 32)) / np.sqrt(32)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, 16).astype(np.float32)
    r = O.route(c, x, wg, b)
    for t in range(64):
        gs, groups, experts = _brute_route(c, r.sb[t])
        assert np.array_equal(np.float32(gs), r.group_scores[t])
        assert set(r.kept_groups[t].tolist()) == groups
        assert set(r.idx[t].tolist()) == experts
        # descending selection score order
        assert (np.diff(r.sb[t][r.idx[t]].astype(np.float64)) <= 0).all()


def test_special_case_single_group_is_plain_topk():
    rng = np.random.default_rng(14)
    c = cfg(E=32, G=1, Gk=1, K=6)
    z = rng.standard_normal((50, 32)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, 32).astype(np.float32)
    r = O.route_from_logits(c, z, b)
    s = scipy.special.expit(z.astype(np.float64)).astype(np.float32)
    for t in range(50):
        sb = [float(np.float32(s[t, e] + b[e])) for e in range(32)]
        ref = sorted(range(32), key=lambda e: (-sb[e], e))[:6]
        assert r.idx[t].tolist() == ref


def test_special_case_zero_bias_is_topk_of_logits():
    rng = np.random.default_rng(15)
    c = cfg(E=64, G=1, Gk=1, K=8)
    z = rng.standard_normal((40, 64)).astype(np.float32) * 3
    r = O.route_from_logits(c, z, np.zeros(64, np.float32))
    for t in range(40):
        assert set(r.idx[t].tolist()) == set(np.argsort(-z[t].astype(np.float64))[:8].tolist())


def test_special_cases_weights():
    # one expert: weight is the route scale exactly
    r = O.route_from_logits(cfg(E=1, G=1, Gk=1, K=1), np.float32([[0.3], [-2.0]]), np.float32([0.05]))
    assert r.w[:, 0].tolist() == [2.5, 2.5]
    # K = E, one group, scale 1: weights are s / sum(s), summing to 1
    rng = np.random.default_rng(16)
    z = rng.standard_normal((10, 8)).astype(np.float32)
    r = O.route_from_logits(cfg(E=8, G=1, Gk=1, K=8, scale=1.0), z, np.zeros(8, np.float32))
    s = scipy.special.expit(z.astype(np.float64))
    ref = np.take_along_axis(s / s.sum(1, keepdims=True), r.idx.astype(np.int64), 1)
    assert np.allclose(r.w, ref, rtol=3e-7, atol=0)


def test_invariants_full_router_shape():
    """256 experts, 8 groups, top-4 groups, top-8 experts (router page summary)."""
    rng = np.random.default_rng(17)
    c = cfg(E=256, G=8, Gk=4, K=8)
    z = rng.standard_normal((2000, 256)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, 256).astype(np.float32)
    r = O.route_from_logits(c, z, b)
    assert r.idx.dtype == np.int32 and r.w.dtype == np.float32
    for t in range(2000):
        assert len(set(r.idx[t].tolist())) == 8
        assert len(set((r.idx[t] // 32).tolist())) <= 4
        assert set((r.idx[t] // 32).tolist()) <= set(r.kept_groups[t].tolist())
    assert (r.w > 0).all()
    assert np.abs(r.w.astype(np.float64).sum(1) - 2.5).max() <= 1e-6
    gmat = O.dense_gate(r, 256)
    assert ((gmat == 0).sum(1) == 248).all()
    # selection never depends on the group order of equal-score experts outside kept groups
    assert np.isneginf(r.masked).sum(1).tolist() == [128] * 2000


def test_token_permutation_equivariance():
    rng = np.random.default_rng(18)
    c = cfg(E=64, G=8, Gk=3, K=6)
    x = rng.standard_normal((100, 48)).astype(np.float32)
    wg = (rng.standard_normal((64, 48)) / 7).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, 64).astype(np.float32)
    p = rng.permutation(100)
    r = O.route(c, x, wg, b)
    rp = O.route(c, x[p], wg, b)
    assert np.array_equal(rp.idx, r.idx[p]) and np.array_equal(rp.w, r.w[p])


def test_near_tie_flags():
    c = cfg(E=8, G=4, Gk=2, K=2)
    # experts 0 and 1 tie exactly inside the chosen pair; group and boundary gaps are wide
    z = np.float32([[1.0, 1.0, -2.0, -2.0, -3.0, -3.0, -4.0, -4.0]])
    r = O.route_from_logits(c, z, np.zeros(8, np.float32))
    nt = O.near_ties(c, r)
    assert nt.order[0] and not nt.group[0] and not nt.boundary[0]
    z2 = np.float32([[3.0, -5.0, 2.0, -2.0, -1.0, -1.0, -1.0, -1.0]])
    r2 = O.route_from_logits(c, z2, np.zeros(8, np.float32))
    assert not O.near_ties(c, r2).any[0]
    assert O.near_ties(c, r2, thresh=10.0).any[0]


# ------------------------------------------------------------------ dispatch

def _rand_idx(rng, t, e, k):
    return np.stack([rng.choice(e, k, replace=False) for _ in range(t)]).astype(np.int32)


@pytest.mark.parametrize("t,e,k", [(1, 16, 4), (37, 16, 4), (300, 256, 8), (0, 8, 2)])
def test_dispatch_vs_lexsort(t, e, k):
    rng = np.random.default_rng(19 + t)
    idx = _rand_idx(rng, t, e, k) if t else np.zeros((0, k), np.int32)
    counts, offsets, row_token, row_of = O.dispatch(idx, e)
    ex = idx.reshape(-1).astype(np.int64)
    tok = np.repeat(np.arange(t), k)
    order = np.lexsort((tok, ex))               # primary key expert, secondary token
    assert np.array_equal(row_token, tok[order])
    assert np.array_equal(counts, np.bincount(ex, minlength=e))
    assert offsets[0] == 0 and offsets[-1] == t * k
    assert np.array_equal(np.diff(offsets), counts)
    # row_of is the inverse permutation
    assert sorted(row_of.reshape(-1).tolist()) == list(range(t * k))
    for tt in range(t):
        for j in range(k):
            row = row_of[tt, j]
            assert row_token[row] == tt and offsets[idx[tt, j]] <= row < offsets[idx[tt, j] + 1]


# ---- softmax scoring (the Gate.forward excerpt's softmax branch; reading R13)
def scfg(**kw):
    c = cfg(**kw)
    c.score_func = "softmax"
    return c


def test_softmax_scores_match_scipy():
    rng = np.random.default_rng(40)
    z = (rng.standard_normal((200, 64)) * 3).astype(np.float32)
    r = O.route_from_logits(scfg(E=64, G=1, Gk=1, K=8), z, None)
    ref = scipy.special.softmax(z.astype(np.float64), axis=1).astype(np.float32)
    ulps = np.abs(r.s.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1 and (ulps > 0).mean() < 0.01


def test_softmax_weights_are_gathered_scores_times_scale():
    rng = np.random.default_rng(41)
    z = rng.standard_normal((30, 16)).astype(np.float32)
    # every expert chosen, scale 1: the weights are the whole distribution and sum to one
    r = O.route_from_logits(scfg(E=16, G=1, Gk=1, K=16, scale=1.0), z, None)
    assert np.allclose(r.w.astype(np.float64).sum(1), 1.0, rtol=0, atol=4e-7)
    # K < E: the gathered scores times the scale, one rounding, no renormalisation
    r = O.route_from_logits(scfg(E=16, G=1, Gk=1, K=4, scale=2.5), z, None)
    gathered = np.take_along_axis(r.s, r.idx.astype(np.int64), 1)
    assert np.array_equal(r.w, (gathered * np.float32(2.5)).astype(np.float32))
    assert (r.w.astype(np.float64).sum(1) < 2.5).all()


def test_softmax_no_bias_single_group_is_topk_of_logits():
    rng = np.random.default_rng(42)
    z = rng.standard_normal((60, 32)).astype(np.float32) * 2
    r = O.route_from_logits(scfg(E=32, G=1, Gk=1, K=6), z, None)
    for t in range(60):
        ref = sorted(range(32), key=lambda e: (-float(z[t, e]), e))[:6]
        assert r.idx[t].tolist() == ref


def test_softmax_shift_invariance():
    """Logits on a 1/256 grid: z + 1 is exact in fp32, z - max z is unchanged, so the scores and
    the routing are bit-identical."""
    rng = np.random.default_rng(43)
    z = (np.round(rng.standard_normal((40, 16)) * 256) / 256).astype(np.float32)
    b = rng.uniform(-0.01, 0.01, 16).astype(np.float32)
    c = scfg(E=16, G=4, Gk=2, K=4)
    r0, r1 = O.route_from_logits(c, z, b), O.route_from_logits(c, z + np.float32(1.0), b)
    assert np.array_equal(r0.s, r1.s) and np.array_equal(r0.idx, r1.idx) and np.array_equal(r0.w, r1.w)


def test_softmax_group_max_brute_force():
    """No bias (group score = the group's best score): the kept groups maximise the sum of group
    maxima over all C(4, 2) group pairs, and the chosen experts maximise the sum of scores over all
    4-subsets of the kept groups' experts."""
    rng = np.random.default_rng(44)
    c = scfg(E=16, G=4, Gk=2, K=4)
    z = rng.standard_normal((64, 16)).astype(np.float32)
    r = O.route_from_logits(c, z, None)
    s = r.s.astype(np.float64)
    for t in range(64):
        gmax = [s[t, 4 * g:4 * g + 4].max() for g in range(4)]
        best_pair = max(itertools.combinations(range(4), 2), key=lambda p: sum(gmax[g] for g in p))
        assert set(r.kept_groups[t].tolist()) == set(best_pair)
        pool = [e for g in best_pair for e in range(4 * g, 4 * g + 4)]
        best = max(itertools.combinations(pool, 4), key=lambda q: sum(s[t, e] for e in q))
        assert set(r.idx[t].tolist()) == set(best)

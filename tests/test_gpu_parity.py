"""Parity of the HIP path (through the C ABI) with the CPU oracle, on seeded synthetic inputs.

Small shapes are checked on every token and span several tiles with ragged tails. The full
DeepSeek-V3 shapes are checked in the launch configuration the bench times: routing and dispatch
on every token; outputs on every token at 16 and 4096 tokens (decode, prefill, skewed), and at
16384 fp8 tokens on a sample holding a row of every 128-row M-tile of every expert (each expert's
ragged last tile by its last row) and of the shared expert. Every compared token is held to the
tolerance on its own as well as in aggregate."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_14_amd import inputs, moe
from oracle import moe_oracle as O
from tests.oracle_io import bias_np, exact, oracle_forward
from tests.parity import dispatch_check, np_i32, out_check, route_check, say, tile_tokens, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
S = inputs.MoeShape

SMALL = {
    "tiny_fp32": inputs.WORKLOADS["tiny_fp32"],
    "ragged_fp32": S("ragged_fp32", tokens=37, dim=100, n_experts=12, n_groups=3, topk_groups=2, topk=3, inter=40,
                     n_shared=2, route_scale=1.5, dtype="f32"),
    "mid_bf16": S("mid_bf16", tokens=300, dim=1024, n_experts=64, n_groups=8, topk_groups=4, topk=8, inter=160,
                  n_shared=1, route_scale=2.5, dtype="bf16"),
    "mid_bf16_shared2": S("mid_bf16_shared2", tokens=77, dim=512, n_experts=32, n_groups=4, topk_groups=2, topk=6,
                          inter=96, n_shared=2, route_scale=2.5, dtype="bf16", hot_bias=0.5),
    "mid_fp8": S("mid_fp8", tokens=200, dim=1024, n_experts=32, n_groups=4, topk_groups=2, topk=6, inter=256,
                 n_shared=1, route_scale=2.5, dtype="fp8"),
    # two shared experts (hidden 2 * inter) in fp8: the 128-row fp8 kernels (the weight-stream ones
    # need the shared hidden size equal to inter), skewed routing with ragged tiles
    "mid_fp8_shared2": S("mid_fp8_shared2", tokens=300, dim=512, n_experts=16, n_groups=4, topk_groups=2, topk=4,
                         inter=512, n_shared=2, route_scale=2.5, dtype="fp8", hot_bias=0.5),
    # the fp8 weight-stream GEMMs (dim and inter multiples of 512): skewed routing gives experts of
    # several M-tiles, ragged tails and empty experts; the second shape runs the k loop's body
    "wstream_fp8": S("wstream_fp8", tokens=600, dim=1024, n_experts=16, n_groups=4, topk_groups=2, topk=4,
                     inter=512, n_shared=1, route_scale=2.5, dtype="fp8", hot_bias=0.5),
    "wstream_fp8_long": S("wstream_fp8_long", tokens=300, dim=2048, n_experts=8, n_groups=2, topk_groups=1,
                          topk=2, inter=1024, n_shared=1, route_scale=2.5, dtype="fp8"),
    # experts of 12+ M-tiles and a 24-tile shared expert: the grouped item order of the 128-row
    # kernels (groups of 6 to 11 M-tiles), checked on every token
    "big_expert_bf16": S("big_expert_bf16", tokens=3000, dim=256, n_experts=2, n_groups=1, topk_groups=1, topk=1,
                         inter=256, n_shared=1, route_scale=1.0, dtype="bf16"),
    "big_expert_fp8": S("big_expert_fp8", tokens=3000, dim=512, n_experts=2, n_groups=1, topk_groups=1, topk=1,
                        inter=512, n_shared=1, route_scale=1.0, dtype="fp8"),
    "wide_bf16": S("wide_bf16", tokens=700, dim=768, n_experts=16, n_groups=4, topk_groups=2, topk=4, inter=256,
                   n_shared=1, route_scale=2.5, dtype="bf16", hot_bias=0.5),
    # more experts than threads in a block: several experts per router thread
    "many_experts_bf16": S("many_experts_bf16", tokens=300, dim=256, n_experts=512, n_groups=16, topk_groups=4,
                           topk=8, inter=64, n_shared=1, route_scale=2.5, dtype="bf16"),
    "max_experts_bf16": S("max_experts_bf16", tokens=40, dim=256, n_experts=1024, n_groups=64, topk_groups=8,
                          topk=16, inter=32, n_shared=1, route_scale=1.0, dtype="bf16"),
    # the router's other branches: softmax scoring (a wave per token here), softmax without bias
    # (groups scored by their best expert; a block per token), one group (plain top-k)
    "softmax_bf16": S("softmax_bf16", tokens=300, dim=512, n_experts=64, n_groups=8, topk_groups=4, topk=8,
                      inter=256, n_shared=1, route_scale=2.5, dtype="bf16", score_func="softmax"),
    "softmax_groupmax_bf16": S("softmax_groupmax_bf16", tokens=200, dim=512, n_experts=64, n_groups=8,
                               topk_groups=3, topk=6, inter=128, n_shared=1, route_scale=1.0, dtype="bf16",
                               has_bias=False, score_func="softmax"),
    "single_group_bf16": S("single_group_bf16", tokens=280, dim=256, n_experts=32, n_groups=1, topk_groups=1,
                           topk=6, inter=96, n_shared=1, route_scale=2.5, dtype="bf16"),
    "softmax_single_group_f32": S("softmax_single_group_f32", tokens=50, dim=128, n_experts=16, n_groups=1,
                                  topk_groups=1, topk=4, inter=64, n_shared=1, route_scale=1.0, dtype="f32",
                                  has_bias=False, score_func="softmax"),
}
FULL = ["decode_bf16", "prefill_bf16", "skewed_bf16", "prefill_fp8"]


def run_block(tens, tokens=None):
    t = tens.shape.tokens if tokens is None else tokens
    blk = moe.Block(tens, max(t, 1))
    out = blk.forward(tens.x[:t])
    torch.cuda.synchronize()
    return blk, out


def gpu_route(blk, shape, T):
    K = shape.topk
    gidx = np_i32(blk.ws_view(T, "idx", torch.int32, T * K).view(T, K))
    gw = blk.ws_view(T, "w", torch.float32, T * K).view(T, K).cpu().numpy()
    return gidx, gw


def gpu_dispatch(blk, shape, T):
    E, R = shape.n_experts, T * shape.topk
    v = lambda n, c: np_i32(blk.ws_view(T, n, torch.int32, c))  # noqa: E731
    return v("counts", E), v("offsets", E + 1), v("row_token", R), v("row_of", R)


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small_all_tokens(name):
    shape = SMALL[name]
    say(f"[forward/small] {name} T={shape.tokens} D={shape.dim} E={shape.n_experts} dtype={shape.dtype}")
    tens = inputs.generate(shape, seed=0, device=DEV)
    blk, out = run_block(tens)
    f = oracle_forward(tens)
    gidx, gw = gpu_route(blk, shape, shape.tokens)
    bad, rep = route_check(shape, f.route, gidx, gw)
    dispatch_check(shape, gidx, *gpu_dispatch(blk, shape, shape.tokens))
    orep = out_check(shape, to_np(out), f.out, skip=bad)
    say(f"  route {rep}\n  out {orep}")


@pytest.mark.parametrize("name", FULL)
def test_forward_full_shape(name):
    shape = inputs.WORKLOADS[name]
    T = shape.tokens
    say(f"[forward/full] {name} T={T} dtype={shape.dtype}: generating weights")
    tens = inputs.generate(shape, seed=0, device=DEV)
    say("  running the block")
    blk, out = run_block(tens)
    say("  oracle routing on every token")
    r = O.route(shape, exact(tens.x), exact(tens.w_gate), bias_np(tens))
    gidx, gw = gpu_route(blk, shape, T)
    bad, rep = route_check(shape, r, gidx, gw)
    say(f"  route {rep}")
    counts, offsets, row_token, _ = gpu_dispatch(blk, shape, T)
    dispatch_check(shape, gidx, counts, offsets, row_token, gpu_dispatch(blk, shape, T)[3])
    if T <= 4096:
        sample = np.arange(T)
    else:  # a row of every 128-row M-tile the fp8 GEMMs ran
        sample = tile_tokens(T, counts, offsets, row_token, 128, np.random.default_rng(1))
    say(f"  oracle forward on {len(sample)} tokens")
    f = oracle_forward(tens, x=exact(tens.x)[sample])
    orep = out_check(shape, to_np(out)[sample], f.out, skip=bad[sample])
    say(f"  out {orep}")
    if name == "skewed_bf16":
        hot = np.isin(r.idx, np.arange(0, shape.n_experts, 8)).mean()
        say(f"  fraction of assignments on the 32 biased experts: {hot:.4f}")


@pytest.mark.parametrize("T,score_func,has_bias", [(16, "softmax", True), (4096, "softmax", True),
                                                   (4096, "sigmoid", False)])
def test_forward_full_shape_router_variants(T, score_func, has_bias):
    """The router branches DeepSeek-V3 does not use, on the full bf16 block: softmax scoring (a
    256-thread block per token at 16 tokens, a wave per token at 4096) and no selection bias
    (groups scored by their best expert). Routing on every token, outputs on sampled tokens."""
    shape = inputs.WORKLOADS["prefill_bf16"].replace(name=f"{score_func}_full_bf16", tokens=T,
                                                     score_func=score_func, has_bias=has_bias)
    say(f"[forward/full router variant] T={T} {score_func} bias={has_bias}")
    tens = inputs.generate(shape, seed=10, device=DEV)
    blk, out = run_block(tens)
    r = O.route(shape, exact(tens.x), exact(tens.w_gate), bias_np(tens))
    gidx, gw = gpu_route(blk, shape, T)
    bad, rep = route_check(shape, r, gidx, gw)
    dispatch_check(shape, gidx, *gpu_dispatch(blk, shape, T))
    sample = np.arange(T) if T <= 16 else np.unique(np.concatenate([[0, T - 1],
                                                                    np.random.default_rng(10).choice(T, 8, replace=False)]))
    f = oracle_forward(tens, x=exact(tens.x)[sample])
    say(f"  route {rep}\n  out {out_check(shape, to_np(out)[sample], f.out, skip=bad[sample])}")


@pytest.mark.parametrize("name", ["decode_bf16", "prefill_fp8"])
def test_forward_full_shape_single_token(name):
    """One token through the full block (batch-1 decode): nine expert M-tiles of one row each on the
    16-row paths (bf16 stream kernels; fp8 16-row kernels), every value checked."""
    shape = inputs.WORKLOADS[name].with_tokens(1)
    say(f"[forward/full, 1 token] {name}")
    tens = inputs.generate(shape, seed=8, device=DEV)
    blk, out = run_block(tens)
    f = oracle_forward(tens)
    gidx, gw = gpu_route(blk, shape, 1)
    bad, rep = route_check(shape, f.route, gidx, gw)
    dispatch_check(shape, gidx, *gpu_dispatch(blk, shape, 1))
    say(f"  route {rep}\n  out {out_check(shape, to_np(out), f.out, skip=bad)}")


@pytest.mark.parametrize("name,T", [("prefill_bf16", 152_000), ("prefill_fp8", 300_000)])
def test_forward_beyond_2gb_activations(name, T):
    """The full block with activations past the 2 GB byte range of the weight-stream kernels'
    buffer resources: bf16 at 152,000 tokens (x is 2.18 GB; the 256-row ring kernels take the
    expert GEMMs, 1.2 M routed rows, 17 GB of expert outputs), fp8 at 300,000 tokens (x's e4m3
    image is 2.15 GB; the 128-row fp8 kernels take them, 34 GB of expert outputs). Routing and
    dispatch on every token, outputs on sampled tokens."""
    shape = inputs.WORKLOADS[name].with_tokens(T)
    assert T * shape.dim * (2 if shape.dtype == "bf16" else 1) > 2 ** 31
    say(f"[forward/beyond 2 GB] {name} T={T}: generating weights")
    tens = inputs.generate(shape, seed=4, device=DEV)
    say("  running the block")
    blk, out = run_block(tens)
    say("  oracle routing on every token")
    xe = exact(tens.x)
    r = O.route(shape, xe, exact(tens.w_gate), bias_np(tens))
    gidx, gw = gpu_route(blk, shape, T)
    bad, rep = route_check(shape, r, gidx, gw)
    say(f"  route {rep}")
    counts, offsets, row_token, row_of = gpu_dispatch(blk, shape, T)
    dispatch_check(shape, gidx, counts, offsets, row_token, row_of)
    # each expert's first, middle and last (ragged) M-tile of the kernels that run here (256-row
    # ring tiles in bf16, 128-row tiles in fp8), every fourth shared-expert M-tile, and tokens
    # whose x row starts past the 2 GB byte offset
    rng = np.random.default_rng(4)
    bm = 256 if shape.dtype == "bf16" else 128
    past = (2 ** 31) // (shape.dim * (2 if shape.dtype == "bf16" else 1)) + 1
    sample = np.unique(np.concatenate([
        tile_tokens(T, counts, offsets, row_token, bm, rng, per_expert="ends", shared_stride=4),
        rng.integers(past, T, 16)]))
    say(f"  oracle forward on {len(sample)} tokens")
    f = oracle_forward(tens, x=xe[sample])
    got = to_np(out[torch.as_tensor(sample, device=out.device)])
    say(f"  out {out_check(shape, got, f.out, skip=bad[sample])}")


@pytest.mark.parametrize("T", [129, 193, 256, 257])
def test_paired_tiles_every_expert_all_tokens(T):
    """Every token takes all 4 experts (top-4 of 4), so each routed expert and the shared expert
    have exactly T rows: the bf16 gate/up kernel's 256-row tiles as 128-row halves at their edges
    (a second half of 1 or 65 rows, two full halves, a full pair and a 1-row tile), every token."""
    shape = S("pair_edges_bf16", tokens=T, dim=256, n_experts=4, n_groups=1, topk_groups=1, topk=4, inter=256,
              n_shared=1, route_scale=1.0, dtype="bf16")
    say(f"[forward/paired tiles] T={T}")
    tens = inputs.generate(shape, seed=13, device=DEV)
    blk, out = run_block(tens)
    f = oracle_forward(tens)
    gidx, gw = gpu_route(blk, shape, T)
    bad, rep = route_check(shape, f.route, gidx, gw)
    counts = gpu_dispatch(blk, shape, T)[0]
    assert (counts == T).all()
    say(f"  route {rep}\n  out {out_check(shape, to_np(out), f.out, skip=bad)}")


@pytest.mark.parametrize("name,T", [("mid_bf16", 1), ("mid_bf16", 17), ("mid_bf16", 64), ("mid_fp8", 3),
                                    ("mid_fp8", 40), ("mid_fp8", 129), ("wstream_fp8", 64),
                                    ("wstream_fp8", 257)])
def test_token_counts_edges(name, T):
    shape = SMALL[name].with_tokens(T)
    say(f"[edges] {name} T={T}")
    tens = inputs.generate(shape, seed=2, device=DEV)
    blk, out = run_block(tens)
    f = oracle_forward(tens)
    gidx, gw = gpu_route(blk, shape, T)
    bad, _ = route_check(shape, f.route, gidx, gw)
    out_check(shape, to_np(out), f.out, skip=bad)


def test_zero_tokens_is_noop():
    shape = SMALL["mid_bf16"]
    tens = inputs.generate(shape.with_tokens(4), seed=0, device=DEV)
    blk = moe.Block(tens, 4)
    out = torch.full_like(tens.x, 7.0)
    moe.forward(blk.cfg, blk.wts, tens.x, out, blk.ws, tokens=0)
    torch.cuda.synchronize()
    assert (out == 7.0).all()


def test_all_tokens_forced_into_one_group():
    """+10 on every expert of group 3: that group is kept by every token and all K experts
    (K <= group size) come from it."""
    shape = SMALL["mid_bf16"]
    tens = inputs.generate(shape, seed=3, device=DEV)
    gs = shape.n_experts // shape.n_groups
    tens.bias[3 * gs:4 * gs] += 10.0
    blk, out = run_block(tens)
    f = oracle_forward(tens)
    gidx, gw = gpu_route(blk, shape, shape.tokens)
    route_check(shape, f.route, gidx, gw)
    assert ((gidx >= 3 * gs) & (gidx < 4 * gs)).all()
    counts = gpu_dispatch(blk, shape, shape.tokens)[0]
    assert (counts == 0).sum() >= shape.n_experts - gs
    out_check(shape, to_np(out), f.out)


def test_route_without_bias_uses_group_max():
    """The excerpt's no-bias branch (bias NULL): groups scored by their best expert."""
    shape = SMALL["mid_bf16"].replace(has_bias=False)
    tens = inputs.generate(shape, seed=4, device=DEV)
    cfg = moe.config(shape)
    T, K = shape.tokens, shape.topk
    ws = torch.empty(moe.workspace_size(cfg, T), dtype=torch.uint8, device=DEV)
    idx = torch.empty(T, K, dtype=torch.int32, device=DEV)
    w = torch.empty(T, K, dtype=torch.float32, device=DEV)
    moe.route(cfg, tens.w_gate, None, tens.x, idx, w, ws)
    torch.cuda.synchronize()
    r = O.route(shape, exact(tens.x), exact(tens.w_gate), None)
    route_check(shape, r, np_i32(idx), w.cpu().numpy())


def _route_only(shape, tens):
    cfg = moe.config(shape)
    T, K = shape.tokens, shape.topk
    ws = torch.empty(moe.workspace_size(cfg, T), dtype=torch.uint8, device=DEV)
    idx = torch.empty(T, K, dtype=torch.int32, device=DEV)
    w = torch.empty(T, K, dtype=torch.float32, device=DEV)
    moe.route(cfg, tens.w_gate, tens.bias, tens.x, idx, w, ws)
    torch.cuda.synchronize()
    return np_i32(idx), w.cpu().numpy()


@pytest.mark.parametrize("T", [40, 300])
def test_route_exact_ties_take_the_lower_index(T):
    """Experts with bit-identical scores (duplicated router rows and biases) are ordered by index:
    pairs held by one lane (e, e + 64) and by neighbouring lanes (e, e + 1), in a block per token
    (40 tokens) and a wave per token (300). Every token must match the oracle exactly."""
    shape = inputs.WORKLOADS["decode_bf16"].replace(name="ties", tokens=T, dim=256, inter=64)
    say(f"[route/exact ties] T={T}")
    tens = inputs.generate(shape, seed=21, device=DEV)
    wg, b = tens.w_gate, tens.bias
    wg[64:128] = wg[0:64]          # same lane, next slot
    b[64:128] = b[0:64]
    wg[129:192:2] = wg[128:192:2]  # neighbouring lanes, same group
    b[129:192:2] = b[128:192:2]
    gi, gw = _route_only(shape, tens)
    r = O.route(shape, exact(tens.x), exact(wg), bias_np(tens))
    both = sum(int(np.isin([e, e + 64], r.idx[t]).all()) for t in range(T) for e in range(64))
    assert both > 0, "no token chose both experts of a tied pair"
    assert (gi == r.idx).all(), f"{int((gi != r.idx).any(axis=1).sum())} tokens differ"
    _, rep = route_check(shape, r, gi, gw)
    say(f"  tokens holding a same-lane tied pair: {both}; {rep}")


@pytest.mark.parametrize("T", [40, 300])
@pytest.mark.parametrize("E,G,Gk,K", [(64, 1, 1, 6), (128, 2, 1, 8), (32, 16, 4, 6), (256, 16, 6, 8)])
def test_route_group_sizes(T, E, G, Gk, K):
    """Group scores for every power-of-two group size the lane steps handle (64, 64, 2, 16 experts
    per group), with a block per token (40 tokens) and a wave per token (300)."""
    shape = inputs.WORKLOADS["decode_bf16"].replace(name=f"groups_{E}x{G}", tokens=T, dim=256, inter=64,
                                                    n_experts=E, n_groups=G, topk_groups=Gk, topk=K)
    say(f"[route/group sizes] T={T} E={E} G={G}")
    tens = inputs.generate(shape, seed=22, device=DEV)
    gi, gw = _route_only(shape, tens)
    r = O.route(shape, exact(tens.x), exact(tens.w_gate), bias_np(tens))
    _, rep = route_check(shape, r, gi, gw)
    say(f"  {rep}")


@pytest.mark.parametrize("T,D,E,G,Gk,K", [(4000, 7168, 256, 8, 4, 8), (1100, 1152, 72, 8, 4, 6),
                                           (1024, 512, 320, 8, 4, 8)])
def test_route_large_batch_tiles(T, D, E, G, Gk, K):
    """moe_route on the large-batch logits tiles (64 tokens x 256 experts, 64-k stages through
    LDS) at their edges: k-slices of an odd number of 32-k chunks, whose last stage is half empty
    (the full router at 4000 tokens: 5 slices of 45 chunks and one of 44; 1152 dims: 8 slices of 5
    chunks and a last of 1), a last token tile partly filled, and expert counts that leave part of
    an expert tile empty (72; 320 = one full tile and one of 64). Routing on every token."""
    shape = inputs.WORKLOADS["prefill_bf16"].replace(name=f"route_{T}x{D}x{E}", tokens=T, dim=D, n_experts=E,
                                                     n_groups=G, topk_groups=Gk, topk=K, inter=128)
    say(f"[route/large batch] T={T} D={D} E={E}")
    tens = inputs.generate(shape, seed=12, device=DEV)
    cfg = moe.config(shape)
    ws = torch.empty(moe.workspace_size(cfg, T), dtype=torch.uint8, device=DEV)
    idx = torch.empty(T, K, dtype=torch.int32, device=DEV)
    w = torch.empty(T, K, dtype=torch.float32, device=DEV)
    moe.route(cfg, tens.w_gate, tens.bias, tens.x, idx, w, ws)
    torch.cuda.synchronize()
    r = O.route(shape, exact(tens.x), exact(tens.w_gate), bias_np(tens))
    _, rep = route_check(shape, r, np_i32(idx), w.cpu().numpy())
    say(f"  route {rep}")


@pytest.mark.parametrize("T,E,K", [(1, 256, 8), (1000, 256, 8), (3000, 64, 6), (513, 16, 4)])
def test_dispatch_standalone(T, E, K):
    shape = inputs.WORKLOADS["decode_bf16"].replace(n_experts=E, topk=K, n_groups=8 if E >= 64 else 4,
                                                    topk_groups=4 if E >= 64 else 2)
    rng = np.random.default_rng(T)
    if E == 256:  # heavy skew: half the assignments on 8 experts
        hot = rng.choice(E, 8, replace=False)
        idx = np.stack([np.concatenate([rng.choice(hot, K // 2, replace=False),
                                        rng.choice(np.setdiff1d(np.arange(E), hot), K - K // 2, replace=False)])
                        for _ in range(T)])
    else:
        idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    cfg = moe.config(shape)
    gi = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    row_token = torch.empty(T * K, dtype=torch.int32, device=DEV)
    row_of = torch.empty(T, K, dtype=torch.int32, device=DEV)
    ws = torch.empty(moe.workspace_size(cfg, T), dtype=torch.uint8, device=DEV)
    moe.dispatch(cfg, gi, counts, offsets, row_token, row_of, ws)
    torch.cuda.synchronize()
    dispatch_check(shape, idx, np_i32(counts), np_i32(offsets), np_i32(row_token), np_i32(row_of))


def test_fp8_activation_codes_bit_exact():
    shape = SMALL["mid_fp8"]
    tens = inputs.generate(shape, seed=5, device=DEV)
    blk, _ = run_block(tens)
    T, D = shape.tokens, shape.dim
    xq = blk.ws_view(T, "xq", torch.uint8, T * D).view(T, D).cpu().numpy()
    sx = blk.ws_view(T, "x_scale", torch.float32, T * D // 128).view(T, D // 128).cpu().numpy()
    q, sc = O.quant_1x128(exact(tens.x).astype(np.float32))
    assert np.array_equal(sx, sc)
    assert np.array_equal(O.e4m3_decode(xq), O.e4m3_decode(q))


def test_fp8_special_blocks():
    """Planted 1x128 blocks: token 0 all zeros (every x and h block has amax 0, so scale 1 and zero
    codes; its output is exactly zero), token 1 one zero block and one block scaled to about 1e3,
    token 2 a single non-zero value. Codes and scales bit-exact, the output within the fp8
    tolerance."""
    shape = SMALL["mid_fp8"]
    tens = inputs.generate(shape, seed=9, device=DEV)
    x = tens.x
    x[0] = 0
    x[1, :128] = 0
    x[1, 256:384] = (x[1, 256:384].float() * 1000).to(x.dtype)
    x[2] = 0
    x[2, 700] = 3.0
    blk, out = run_block(tens)
    T, D = shape.tokens, shape.dim
    xq = blk.ws_view(T, "xq", torch.uint8, T * D).view(T, D).cpu().numpy()
    sx = blk.ws_view(T, "x_scale", torch.float32, T * D // 128).view(T, D // 128).cpu().numpy()
    q, sc = O.quant_1x128(exact(x).astype(np.float32))
    assert np.array_equal(sx, sc) and (sx[0] == 1.0).all() and sx[1, 0] == 1.0
    assert np.array_equal(O.e4m3_decode(xq), O.e4m3_decode(q))
    assert (xq[0] & 0x7F == 0).all()
    f = oracle_forward(tens)
    gidx, gw = gpu_route(blk, shape, T)
    bad, _ = route_check(shape, f.route, gidx, gw)
    got = to_np(out)
    assert (got[0] == 0).all()
    out_check(shape, got, f.out, skip=bad)


@pytest.mark.parametrize("name", ["mid_bf16", "mid_fp8", "wstream_fp8"])
def test_deterministic_reruns(name):
    shape = SMALL[name]
    tens = inputs.generate(shape, seed=6, device=DEV)
    blk = moe.Block(tens, shape.tokens)
    a = blk.forward(tens.x).clone()
    ws_a = blk.ws.clone()
    b = blk.forward(tens.x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    lay = blk.layout(shape.tokens)
    assert torch.equal(ws_a[lay.idx:lay.o_shared], blk.ws[lay.idx:lay.o_shared])


@pytest.mark.parametrize("name", ["decode_bf16", "mid_fp8", "wstream_fp8"])
def test_graph_replay_matches_eager(name):
    """The whole forward captured in a HIP graph (nothing in it allocates or memsets) replays to
    the eager result, every time, with eager launches and synchronisations in between."""
    shape = inputs.WORKLOADS[name] if name in inputs.WORKLOADS else SMALL[name]
    say(f"[graph] {name}")
    tens = inputs.generate(shape, seed=7, device=DEV)
    blk = moe.Block(tens, shape.tokens)
    ref = blk.forward(tens.x).clone()
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        blk.forward(tens.x, out)  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        blk.forward(tens.x, out)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        blk.forward(tens.x)  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["mid_bf16", "wstream_fp8"])
def test_workspace_reuse_across_token_counts(name):
    """One workspace, calls of 300, 17, 1 and again 300 tokens: every output equals the one a fresh
    workspace gives (nothing of an earlier, larger call leaks through the tile lists or counters)."""
    shape = SMALL[name]
    tens = inputs.generate(shape.with_tokens(300), seed=11, device=DEV)
    blk = moe.Block(tens, 300)
    for t in (300, 17, 1, 300):
        out = blk.forward(tens.x[:t])
        fresh = moe.Block(tens, t).forward(tens.x[:t])
        torch.cuda.synchronize()
        assert torch.equal(out, fresh), t


def test_two_streams_two_workspaces():
    """Two blocks with their own workspaces running on two streams at once give the same outputs as
    run one after the other (the library keeps no shared device state between calls)."""
    sa, sb = SMALL["mid_bf16"], SMALL["wstream_fp8"]
    ta = inputs.generate(sa, seed=12, device=DEV)
    tb = inputs.generate(sb, seed=13, device=DEV)
    ba, bb = moe.Block(ta, sa.tokens), moe.Block(tb, sb.tokens)
    ref_a, ref_b = ba.forward(ta.x).clone(), bb.forward(tb.x).clone()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    oa, ob = torch.empty_like(ref_a), torch.empty_like(ref_b)
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s1):
            ba.forward(ta.x, oa)
        with torch.cuda.stream(s2):
            bb.forward(tb.x, ob)
        torch.cuda.synchronize()
        assert torch.equal(oa, ref_a) and torch.equal(ob, ref_b)


def _oracle_h_fp8(tens, rows_tok, rows_exp, e_shared):
    """The oracle's e4m3 codes and 1x128 scales of h for the given (token, expert) rows: h from the
    x image the GEMMs read, W1 and W3 dequantised, rounded to fp32, then requantised (R7, R9)."""
    from tests.oracle_io import expert_fn

    expert, shared = expert_fn(tens)
    xa = O.activation_input(exact(tens.x), "fp8")
    codes = np.empty((len(rows_tok), tens.shape.inter), np.uint8)
    scales = np.empty((len(rows_tok), tens.shape.inter // 128), np.float32)
    for e in np.unique(rows_exp):
        sel = np.nonzero(rows_exp == e)[0]
        w1, w3, _ = shared() if e == e_shared else expert(int(e))
        x = xa[rows_tok[sel]]
        g, u = x @ w1.T, x @ w3.T
        h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
        codes[sel], scales[sel] = O.quant_1x128(h)
    return codes, scales


@pytest.mark.parametrize("name,T", [("wstream_fp8", 600), ("big_expert_fp8", 3000), ("mid_fp8", 200),
                                    ("mid_fp8", 40)])
def test_fp8_h_codes_match_oracle(name, T):
    """The gate/up kernels' fused SwiGLU + requantisation epilogue (weight-stream kernels at 600 and
    3000 tokens, 128-row kernels at 200, 16-row kernels at 40), on every routed and shared row.

    The kernels form h from fp32 sums of exact fp8 products promoted per 128-k block, the oracle
    from an fp64 sum: h differs by up to ~1e-4 of its block's amax. So each 1x128 scale (amax / 448)
    is within 1e-3 relative of the oracle's, and each code's value in scaled units (code value =
    h / scale) is within one e4m3 step of the larger of the two, plus 448 x 1e-4 for the h error
    (which near zero spans several subnormal steps); at least 99% of the codes are equal. A wrong
    scale rule or block shape moves scales by O(1); truncation instead of round-to-nearest-even
    changes about half of the codes."""
    shape = SMALL[name].with_tokens(T)
    K, I = shape.topk, shape.inter
    say(f"[fp8 h codes] {name} T={T}")
    tens = inputs.generate(shape, seed=14, device=DEV)
    blk, _ = run_block(tens)
    R = T * K
    counts, offsets, row_token, _ = gpu_dispatch(blk, shape, T)
    row_exp = np.repeat(np.arange(shape.n_experts), counts)
    hq = np.concatenate([blk.ws_view(T, "h_routed", torch.uint8, R * I).view(R, I).cpu().numpy(),
                         blk.ws_view(T, "h_shared", torch.uint8, T * I).view(T, I).cpu().numpy()])
    hs = np.concatenate([blk.ws_view(T, "h_scale", torch.float32, R * I // 128).view(R, I // 128).cpu().numpy(),
                         blk.ws_view(T, "h_shared_scale", torch.float32, T * I // 128).view(T, I // 128).cpu().numpy()])
    toks = np.concatenate([row_token, np.arange(T)])
    exps = np.concatenate([row_exp, np.full(T, shape.n_experts)])
    oq, osc = _oracle_h_fp8(tens, toks, exps, shape.n_experts)
    rel = np.abs(hs.astype(np.float64) - osc) / osc
    qg, qo = O.e4m3_decode(hq), O.e4m3_decode(oq)
    mag = np.maximum(np.abs(qg), np.abs(qo))
    # one e4m3 step at that magnitude: 2^(e - 3) for normals (e >= -6), 2^-9 below
    ulp = 2.0 ** (np.maximum(np.floor(np.log2(np.maximum(mag, 2.0 ** -9))), -6) - 3)
    excess = np.abs(qg - qo) / (ulp + 448 * 1e-4)
    rep = dict(rows=len(toks), scale_max_rel=float(rel.max()), codes_equal=float((qg == qo).mean()),
               worst_code_diff_over_bound=float(excess.max()))
    say(f"  {rep}")
    assert rel.max() <= 1e-3, rep
    assert excess.max() <= 1.0 and (qg == qo).mean() >= 0.99, rep


@pytest.mark.parametrize("name,T", [("mid_bf16", 40), ("mid_bf16", 300), ("mid_fp8", 200)])
def test_nan_token_still_routes_to_valid_experts(name, T):
    """A token whose x holds a NaN has NaN logits; its selection scores rank below every number, so
    it still gets K distinct experts in [0, E) (the lowest indices of the lowest kept groups) and
    nothing downstream reads outside its buffers. Every other token routes and computes exactly as
    without it (a block per token at 40 tokens, a wave per token at 300)."""
    shape = SMALL[name].with_tokens(T)
    say(f"[nan token] {name} T={T}")
    tens = inputs.generate(shape, seed=15, device=DEV)
    nan_tok = T // 3
    tens.x[nan_tok, 5] = float("nan")
    blk, out = run_block(tens)
    gidx, gw = gpu_route(blk, shape, T)
    assert ((gidx >= 0) & (gidx < shape.n_experts)).all()
    assert all(len(set(r.tolist())) == shape.topk for r in gidx)
    others = np.setdiff1d(np.arange(T), [nan_tok])
    f = oracle_forward(tens, x=exact(tens.x)[others])
    bad, rep = route_check(shape, f.route, gidx[others], gw[others])
    counts, offsets, row_token, row_of = gpu_dispatch(blk, shape, T)
    dispatch_check(shape, gidx, counts, offsets, row_token, row_of)
    got = to_np(out)
    say(f"  route {rep}\n  out {out_check(shape, got[others], f.out, skip=bad)}")


def test_nan_bias_expert_is_never_chosen():
    """A NaN selection bias ranks that expert below every number: routing equals the oracle's with
    that bias at -inf (the expert is never chosen while enough others remain)."""
    shape = SMALL["mid_bf16"]
    tens = inputs.generate(shape, seed=16, device=DEV)
    tens.bias[9] = float("nan")
    blk, out = run_block(tens)
    T = shape.tokens
    gidx, gw = gpu_route(blk, shape, T)
    b = bias_np(tens)
    b[9] = -np.inf
    r = O.route(shape, exact(tens.x), exact(tens.w_gate), b)
    route_check(shape, r, gidx, gw)
    assert not (gidx == 9).any()
    assert np.isfinite(to_np(out)).all()

"""The fused single-launch decode (moe_forward_fused, through the C ABI): the same output as
moe_forward bit for bit (its phases run the separate kernels' device code), the same routing and
dispatch in the workspace, and parity with the oracle, for bf16 blocks of 1 to 32 tokens: the full
DeepSeek-V3 block at decode shape and small shapes with every router branch."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_14_amd import inputs, moe
from tests.oracle_io import oracle_forward
from tests.parity import dispatch_check, np_i32, out_check, route_check, say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
S = inputs.MoeShape

SMALL = {
    "mid_bf16": S("mid_bf16", tokens=32, dim=1024, n_experts=64, n_groups=8, topk_groups=4, topk=8, inter=160,
                  n_shared=1, route_scale=2.5, dtype="bf16"),
    "shared2_bf16": S("shared2_bf16", tokens=20, dim=512, n_experts=32, n_groups=4, topk_groups=2, topk=6, inter=96,
                      n_shared=2, route_scale=2.5, dtype="bf16", hot_bias=0.5),
    "softmax_bf16": S("softmax_bf16", tokens=24, dim=512, n_experts=64, n_groups=8, topk_groups=4, topk=8, inter=256,
                      n_shared=1, route_scale=2.5, dtype="bf16", score_func="softmax"),
    "nobias_bf16": S("nobias_bf16", tokens=17, dim=512, n_experts=64, n_groups=8, topk_groups=3, topk=6, inter=128,
                     n_shared=1, route_scale=1.0, dtype="bf16", has_bias=False),
    "one_group_bf16": S("one_group_bf16", tokens=9, dim=256, n_experts=32, n_groups=1, topk_groups=1, topk=6,
                        inter=96, n_shared=1, route_scale=2.5, dtype="bf16"),
}


def fused_and_plain(tens, T):
    blk = moe.Block(tens, T)
    x = tens.x[:T]
    ref = blk.forward(x)
    torch.cuda.synchronize()
    ws_ref = routing_state(blk, tens.shape, T)
    out = torch.full_like(x, float("nan"))
    blk.ws.fill_(0xAB)  # the fused path must not depend on what the workspace held
    moe.forward_fused(blk.cfg, blk.wts, x, out, blk.ws)
    torch.cuda.synchronize()
    return blk, ref, out, ws_ref


def routing_state(blk, shape, T):
    """idx, w, counts, offsets, row_token and row_of as left in the workspace."""
    R, E = T * shape.topk, shape.n_experts
    parts = [("idx", torch.int32, R), ("w", torch.float32, R), ("counts", torch.int32, E),
             ("offsets", torch.int32, E + 1), ("row_token", torch.int32, R), ("row_of", torch.int32, R)]
    return [blk.ws_view(T, n, dt, c).clone() for n, dt, c in parts]


def gpu_route(blk, shape, T):
    K = shape.topk
    gidx = np_i32(blk.ws_view(T, "idx", torch.int32, T * K).view(T, K))
    gw = blk.ws_view(T, "w", torch.float32, T * K).view(T, K).cpu().numpy()
    return gidx, gw


@pytest.mark.parametrize("name", list(SMALL))
def test_fused_equals_forward_and_oracle_small(name):
    shape = SMALL[name]
    T = shape.tokens
    say(f"[fused/small] {name} T={T}")
    tens = inputs.generate(shape, seed=31, device=DEV)
    blk, ref, out, ws_ref = fused_and_plain(tens, T)
    assert torch.equal(out, ref)
    # routing, weights and the dispatch permutation as the separate kernels left them
    for a, b in zip(routing_state(blk, shape, T), ws_ref):
        assert torch.equal(a, b)
    f = oracle_forward(tens)
    gidx, gw = gpu_route(blk, shape, T)
    bad, rep = route_check(shape, f.route, gidx, gw)
    E, R = shape.n_experts, T * shape.topk
    v = lambda n, c: np_i32(blk.ws_view(T, n, torch.int32, c))  # noqa: E731
    dispatch_check(shape, gidx, v("counts", E), v("offsets", E + 1), v("row_token", R), v("row_of", R))
    say(f"  route {rep}\n  out {out_check(shape, to_np(out), f.out, skip=bad)}")


@pytest.mark.parametrize("T", [16, 1, 5, 32])
def test_fused_equals_forward_full_decode(T):
    """The full DeepSeek-V3 block (dim 7168, 256 experts, 8 groups / top-4 / top-8, inter 2048):
    equal to moe_forward bit for bit, and within the bf16 tolerance of the oracle on every token."""
    shape = inputs.WORKLOADS["decode_bf16"].with_tokens(T)
    say(f"[fused/full] decode_bf16 T={T}")
    tens = inputs.generate(shape, seed=32 + T, device=DEV)
    blk, ref, out, ws_ref = fused_and_plain(tens, T)
    assert torch.equal(out, ref)
    for a, b in zip(routing_state(blk, shape, T), ws_ref):
        assert torch.equal(a, b)
    f = oracle_forward(tens)
    gidx, gw = gpu_route(blk, shape, T)
    bad, rep = route_check(shape, f.route, gidx, gw)
    say(f"  route {rep}\n  out {out_check(shape, to_np(out), f.out, skip=bad)}")


def test_fused_reruns_and_graph_replay():
    """Bit-identical reruns; captured in a HIP graph (a cooperative launch), replayed three times
    with eager work between, each replay equal to the eager result."""
    shape = inputs.WORKLOADS["decode_bf16"]
    tens = inputs.generate(shape, seed=40, device=DEV)
    blk = moe.Block(tens, shape.tokens)
    ref = blk.forward(tens.x).clone()
    out = torch.empty_like(ref)
    for _ in range(3):
        moe.forward_fused(blk.cfg, blk.wts, tens.x, out, blk.ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.forward_fused(blk.cfg, blk.wts, tens.x, out, blk.ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward_fused(blk.cfg, blk.wts, tens.x, out, blk.ws)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        blk.forward(tens.x)
        torch.cuda.synchronize()

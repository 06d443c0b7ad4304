"""Parity of the dense feed-forward (moe_ffn, through the C ABI) with the CPU oracle.

Small shapes are checked on every token at token counts that take each kernel path (16-row
stream / fp8 kernels below 64 tokens, the weight-stream, ring and 128-row kernels above) with
ragged tails whose last 128-row tile has 1, 2, 3 or 4 live 32-row groups (129, 64 / 300, 96 / 200,
128 tokens); the DeepSeek-V3 dense layer (dim 7168, intermediate 18,432) is checked at the
decode, prefill and FP8-prefill token counts on every token (16 and 4096 tokens) or on a token of
every 128-row M-tile (16384 fp8 tokens, and past the kernels' 2 GB range a token of every M-tile
of the kernels that run there). Every compared token is held to the tolerance on its own."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_14_amd import inputs, moe
from tests.oracle_io import exact, ffn_mats, oracle_ffn
from tests.parity import out_check, say, tile_tokens, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
F = inputs.FfnShape

SMALL = {
    "dense_tiny_fp32": inputs.FFN_WORKLOADS["dense_tiny_fp32"],
    # bf16: weight-stream kernels (dim % 256, inter % 256), the ring kernels (inter % 128), the
    # 128-row kernels (dim % 128, inter % 64)
    "dense_wstream_bf16": F("dense_wstream_bf16", tokens=300, dim=512, inter=1536, dtype="bf16"),
    "dense_ring_bf16": F("dense_ring_bf16", tokens=300, dim=512, inter=1408, dtype="bf16"),
    "dense_wide_bf16": F("dense_wide_bf16", tokens=300, dim=384, inter=1472, dtype="bf16"),
    # fp8: weight-stream kernels (dim, inter % 512) and the 128-row kernels
    "dense_wstream_fp8": F("dense_wstream_fp8", tokens=300, dim=1024, inter=1536, dtype="fp8"),
    "dense_wide_fp8": F("dense_wide_fp8", tokens=300, dim=512, inter=640, dtype="fp8"),
}
FULL = ["dense_decode_bf16", "dense_prefill_bf16", "dense_prefill_fp8"]
# 13 M-tiles of 128 rows: two groups (7 + 6) in the grouped item order, every token checked
GROUPED = [F("dense_grouped_bf16", tokens=1664, dim=256, inter=512, dtype="bf16"),
           F("dense_grouped_fp8", tokens=1664, dim=512, inter=512, dtype="fp8")]


def run_ffn(tens, tokens):
    blk = moe.Ffn(tens, max(tokens, 1))
    out = blk.forward(tens.x[:tokens])
    torch.cuda.synchronize()
    return blk, out


@pytest.mark.parametrize("name,T", [(n, t) for n in SMALL for t in (1, 16, 63, 64, 96, 129, 200, 300)])
def test_ffn_small_all_tokens(name, T):
    shape = SMALL[name].with_tokens(T)
    say(f"[ffn/small] {name} T={T} D={shape.dim} I={shape.inter} dtype={shape.dtype}")
    tens = inputs.generate_ffn(shape, seed=0, device=DEV)
    _, out = run_ffn(tens, T)
    rep = out_check(shape, to_np(out), oracle_ffn(tens))
    say(f"  out {rep}")


@pytest.mark.parametrize("T", [128, 129, 192, 193, 256, 257, 384, 385])
def test_ffn_paired_tile_edges(T):
    """The bf16 gate/up kernel takes 256-row tiles as one or two 128-row halves: tiles of exactly
    128 rows (one half), 129 (a second half of one row), 192 / 193 (a second half of 64 / 65 rows,
    where its multiplied row groups round up from 2 to 4), 256 (two full halves) and a last tile of
    1 or 129 rows after full ones. Every token checked."""
    shape = SMALL["dense_wstream_bf16"].with_tokens(T)
    say(f"[ffn/paired edges] T={T}")
    tens = inputs.generate_ffn(shape, seed=6, device=DEV)
    _, out = run_ffn(tens, T)
    say(f"  out {out_check(shape, to_np(out), oracle_ffn(tens))}")


@pytest.mark.parametrize("shape", GROUPED, ids=lambda s: s.name)
def test_ffn_grouped_order_all_tokens(shape):
    say(f"[ffn/grouped] {shape.name} T={shape.tokens}")
    tens = inputs.generate_ffn(shape, seed=5, device=DEV)
    _, out = run_ffn(tens, shape.tokens)
    say(f"  out {out_check(shape, to_np(out), oracle_ffn(tens))}")


@pytest.mark.parametrize("name", FULL)
def test_ffn_full_shape(name):
    shape = inputs.FFN_WORKLOADS[name]
    T = shape.tokens
    say(f"[ffn/full] {name} T={T} D={shape.dim} I={shape.inter} dtype={shape.dtype}: generating weights")
    tens = inputs.generate_ffn(shape, seed=0, device=DEV)
    _, out = run_ffn(tens, T)
    # every token up to 4096; at 16384 (fp8) a token of every 128-row M-tile
    rng = np.random.default_rng(1)
    sample = np.arange(T) if T <= 4096 else tile_tokens(T, [], [0], [], 128, rng)
    say(f"  oracle on {len(sample)} tokens")
    want = oracle_ffn(tens, x=exact(tens.x)[sample], mats=ffn_mats(tens))
    rep = out_check(shape, to_np(out)[sample], want)
    say(f"  out {rep}")


@pytest.mark.parametrize("name", ["dense_decode_bf16", "dense_prefill_fp8"])
def test_ffn_full_width_single_token(name):
    """One token through the 18,432-wide layer (the 16-row paths, every value)."""
    shape = inputs.FFN_WORKLOADS[name].with_tokens(1)
    say(f"[ffn/full, 1 token] {name}")
    tens = inputs.generate_ffn(shape, seed=6, device=DEV)
    _, out = run_ffn(tens, 1)
    say(f"  out {out_check(shape, to_np(out), oracle_ffn(tens, mats=ffn_mats(tens)))}")


@pytest.mark.parametrize("name,T", [("dense_prefill_bf16", 60_000), ("dense_prefill_fp8", 120_000)])
def test_ffn_beyond_2gb_activations(name, T):
    """The 18,432-wide layer with h [T, 18432] past the 2 GB byte range of the weight-stream
    kernels' buffer resources (bf16 h 2.21 GB at 60,000 tokens: the ring kernels run; fp8 h 2.21 GB
    at 120,000 tokens: the 128-row fp8 kernels run), sampled tokens against the oracle."""
    shape = inputs.FFN_WORKLOADS[name].with_tokens(T)
    assert T * shape.inter * (2 if shape.dtype == "bf16" else 1) > 2 ** 31
    say(f"[ffn/beyond 2 GB] {name} T={T}: generating weights")
    tens = inputs.generate_ffn(shape, seed=4, device=DEV)
    _, out = run_ffn(tens, T)
    # a token of every M-tile the kernels ran (256 rows in bf16, 128 in fp8)
    rng = np.random.default_rng(4)
    sample = tile_tokens(T, [], [0], [], 256 if shape.dtype == "bf16" else 128, rng)
    want = oracle_ffn(tens, x=exact(tens.x[torch.as_tensor(sample, device=tens.x.device)]), mats=ffn_mats(tens))
    got = to_np(out[torch.as_tensor(sample, device=out.device)])
    say(f"  out {out_check(shape, got, want)}")


def test_ffn_zero_tokens_is_noop():
    tens = inputs.generate_ffn(SMALL["dense_wstream_bf16"].with_tokens(4), seed=0, device=DEV)
    blk = moe.Ffn(tens, 4)
    out = torch.full_like(tens.x, 7.0)
    moe.ffn(blk.cfg, blk.wts, tens.x, out, blk.ws, tokens=0)
    torch.cuda.synchronize()
    assert (out == 7.0).all()


@pytest.mark.parametrize("name", ["dense_wstream_bf16", "dense_wstream_fp8"])
def test_ffn_deterministic_reruns(name):
    tens = inputs.generate_ffn(SMALL[name], seed=3, device=DEV)
    blk, a = run_ffn(tens, tens.shape.tokens)
    b = blk.forward(tens.x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_ffn_graph_replay_matches_eager():
    """The dense feed-forward captured in a HIP graph replays to the eager result, with eager
    launches and synchronisations between the replays."""
    tens = inputs.generate_ffn(SMALL["dense_wstream_fp8"], seed=7, device=DEV)
    blk = moe.Ffn(tens, tens.shape.tokens)
    ref = blk.forward(tens.x).clone()
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        blk.forward(tens.x, out)
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
        blk.forward(tens.x)
        torch.cuda.synchronize()

"""Seeded synthetic inputs for the DeepSeek-V3-style MoE block.

This module is shared by the CPU oracle tests and by the HIP path. It draws
numbers and stores them in the block's storage dtypes; it holds none of the
block's arithmetic (no routing, no expert FFN, no combine, no activation
quantisation).

Shapes follow the open-model-atlas MoE-block page (DeepSeek-V3.2-Exp, "Mixture
of experts": block input/output [B, T, 7168], parameter table with router
1,835,264, routed/shared expert 44,040,192 each) and the router page (Gate
constructor: weight [n_routed_experts, dim], bias [n_routed_experts] fp32).
Expert matrices use the [out, in] layout of a linear layer:
w1, w3: [E, I, D]; w2: [E, D, I]; shared ws1, ws3: [S, D], ws2: [D, S].

Distributions (no trained weights exist here): x ~ N(0, 1); every weight
matrix ~ N(0, 1/fan_in) with fan_in = D for the router, w1, w3 and fan_in = I
(or S) for w2; bias ~ U(-0.1, 0.1). The skewed workload adds +0.5 to the bias
of the experts e with e % 8 == 0 (32 of 256, four per group of 32).

For the FP8 workload the expert weights are drawn in fp32, then stored as
OCP e4m3fn codes with one fp32 scale per 128x128 block of the [out, in]
matrix (scale = block amax / 448, the cast done by torch's float8 type); the
block's hot path never sees the fp32 values.

Every tensor has its own torch.Generator seeded from (seed, tensor id,
expert), so any one expert can be regenerated alone.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional

import torch


@dataclass(frozen=True)
class MoeShape:
    """One MoE-block workload. Field names follow the Gate/MoE constructors."""

    name: str
    tokens: int
    dim: int
    n_experts: int
    n_groups: int
    topk_groups: int
    topk: int
    inter: int
    n_shared: int
    route_scale: float
    dtype: str  # "f32" | "bf16" | "fp8"
    hot_bias: float = 0.0  # added to the bias of experts e with e % 8 == 0
    has_bias: bool = True
    score_func: str = "sigmoid"  # router scoring: "sigmoid" or "softmax"

    @property
    def shared_inter(self) -> int:
        return self.n_shared * self.inter

    def with_tokens(self, t: int) -> "MoeShape":
        return dataclasses.replace(self, tokens=t)

    def replace(self, **kw) -> "MoeShape":
        return dataclasses.replace(self, **kw)


_FULL = dict(dim=7168, n_experts=256, n_groups=8, topk_groups=4, topk=8, inter=2048,
             n_shared=1, route_scale=2.5)

#: The five workloads. "tiny_fp32" is small enough for the oracle on every
#: token; the others are the full DeepSeek-V3 block at decode, prefill,
#: skewed-prefill and FP8-prefill token counts.
WORKLOADS = {
    "tiny_fp32": MoeShape("tiny_fp32", tokens=64, dim=256, n_experts=16, n_groups=4, topk_groups=2,
                          topk=4, inter=64, n_shared=1, route_scale=2.5, dtype="f32"),
    "decode_bf16": MoeShape("decode_bf16", tokens=16, dtype="bf16", **_FULL),
    "prefill_bf16": MoeShape("prefill_bf16", tokens=4096, dtype="bf16", **_FULL),
    "skewed_bf16": MoeShape("skewed_bf16", tokens=4096, dtype="bf16", hot_bias=0.5, **_FULL),
    "prefill_fp8": MoeShape("prefill_fp8", tokens=16384, dtype="fp8", **_FULL),
}

_TID = dict(x=1, w_gate=2, bias=3, w1=4, w3=5, w2=6, ws1=7, ws3=8, ws2=9)
FP8_BLOCK = 128


def _gen(device, seed: int, tid: int, sub: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + tid * 100_003 + sub) % (2 ** 62))
    return g


def _storage(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


@dataclass
class MoeTensors:
    """Device (or host) tensors of one workload. Scales are None unless fp8."""

    shape: MoeShape
    x: torch.Tensor
    w_gate: torch.Tensor
    bias: Optional[torch.Tensor]
    w1: torch.Tensor
    w3: torch.Tensor
    w2: torch.Tensor
    ws1: torch.Tensor
    ws3: torch.Tensor
    ws2: torch.Tensor
    s1: Optional[torch.Tensor] = None
    s3: Optional[torch.Tensor] = None
    s2: Optional[torch.Tensor] = None
    ss1: Optional[torch.Tensor] = None
    ss3: Optional[torch.Tensor] = None
    ss2: Optional[torch.Tensor] = None


def _normal(rows: int, cols: int, std: float, g: torch.Generator, device) -> torch.Tensor:
    return torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32) * std


def _fp8_blocks(w: torch.Tensor):
    """fp32 [R, C] -> (e4m3fn codes [R, C], fp32 scales [R/128, C/128])."""
    r, c = w.shape
    blk = w.view(r // FP8_BLOCK, FP8_BLOCK, c // FP8_BLOCK, FP8_BLOCK)
    amax = blk.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (blk / scale[:, None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(r, c), scale.contiguous()


def _matrix(shape: MoeShape, seed: int, tid: int, sub: int, rows: int, cols: int, fan_in: int, device):
    w = _normal(rows, cols, fan_in ** -0.5, _gen(device, seed, tid, sub), device)
    if shape.dtype == "fp8":
        return _fp8_blocks(w)
    return w.to(_storage(shape.dtype)), None


def expert_weights(shape: MoeShape, e: int, seed: int = 0, device="cpu"):
    """Regenerate routed expert e alone: (w1, w3, w2, s1, s3, s2)."""
    d, i = shape.dim, shape.inter
    w1, s1 = _matrix(shape, seed, _TID["w1"], e, i, d, d, device)
    w3, s3 = _matrix(shape, seed, _TID["w3"], e, i, d, d, device)
    w2, s2 = _matrix(shape, seed, _TID["w2"], e, d, i, i, device)
    return w1, w3, w2, s1, s3, s2


def generate(shape: MoeShape, seed: int = 0, device="cpu") -> MoeTensors:
    """Draw every input of the block for `shape`. Deterministic per device type."""
    device = torch.device(device)
    t, d, e, i, s = shape.tokens, shape.dim, shape.n_experts, shape.inter, shape.shared_inter
    meta = device.type == "meta"
    act = torch.float32 if shape.dtype == "f32" else torch.bfloat16

    if meta:
        wdt = torch.float8_e4m3fn if shape.dtype == "fp8" else _storage(shape.dtype)
        z = lambda *sz, dt=wdt: torch.empty(*sz, dtype=dt, device=device)  # noqa: E731
        sc = (lambda *sz: torch.empty(*sz, dtype=torch.float32, device=device)) if shape.dtype == "fp8" \
            else (lambda *sz: None)
        b = FP8_BLOCK
        return MoeTensors(shape, x=z(t, d, dt=act), w_gate=z(e, d, dt=act),
                          bias=z(e, dt=torch.float32) if shape.has_bias else None,
                          w1=z(e, i, d), w3=z(e, i, d), w2=z(e, d, i), ws1=z(s, d), ws3=z(s, d), ws2=z(d, s),
                          s1=sc(e, i // b, d // b), s3=sc(e, i // b, d // b), s2=sc(e, d // b, i // b),
                          ss1=sc(s // b, d // b), ss3=sc(s // b, d // b), ss2=sc(d // b, s // b))

    x = torch.randn(t, d, generator=_gen(device, seed, _TID["x"]), device=device, dtype=torch.float32).to(act)
    w_gate = _normal(e, d, d ** -0.5, _gen(device, seed, _TID["w_gate"]), device).to(act)
    bias = None
    if shape.has_bias:
        bias = torch.rand(e, generator=_gen(device, seed, _TID["bias"]), device=device,
                          dtype=torch.float32) * 0.2 - 0.1
        if shape.hot_bias:
            bias[0::8] += shape.hot_bias

    fp8 = shape.dtype == "fp8"
    wdt = torch.float8_e4m3fn if fp8 else _storage(shape.dtype)
    w1 = torch.empty(e, i, d, dtype=wdt, device=device)
    w3 = torch.empty(e, i, d, dtype=wdt, device=device)
    w2 = torch.empty(e, d, i, dtype=wdt, device=device)
    s1 = s3 = s2 = None
    if fp8:
        b = FP8_BLOCK
        s1 = torch.empty(e, i // b, d // b, dtype=torch.float32, device=device)
        s3 = torch.empty_like(s1)
        s2 = torch.empty(e, d // b, i // b, dtype=torch.float32, device=device)
    for ex in range(e):
        a1, a3, a2, c1, c3, c2 = expert_weights(shape, ex, seed, device)
        w1[ex], w3[ex], w2[ex] = a1, a3, a2
        if fp8:
            s1[ex], s3[ex], s2[ex] = c1, c3, c2
    ws1, ss1 = _matrix(shape, seed, _TID["ws1"], 0, s, d, d, device)
    ws3, ss3 = _matrix(shape, seed, _TID["ws3"], 0, s, d, d, device)
    ws2, ss2 = _matrix(shape, seed, _TID["ws2"], 0, d, s, s, device)
    return MoeTensors(shape, x, w_gate, bias, w1, w3, w2, ws1, ws3, ws2, s1, s3, s2, ss1, ss3, ss2)


def regenerate_x(shape: MoeShape, seed: int = 0, device="cpu") -> torch.Tensor:
    """The activations alone (same values as generate(...).x)."""
    act = torch.float32 if shape.dtype == "f32" else torch.bfloat16
    return torch.randn(shape.tokens, shape.dim, generator=_gen(torch.device(device), seed, _TID["x"]),
                       device=device, dtype=torch.float32).to(act)


# --------------------------------------------------------------------------
# Dense feed-forward of the first layers ("Hardware for DeepSeek-V3 and R1",
# section "Why the dense layers and shared expert matter": intermediate 18,432)
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class FfnShape:
    """One dense SwiGLU feed-forward workload: tokens x dim -> inter -> dim."""

    name: str
    tokens: int
    dim: int
    inter: int
    dtype: str  # "f32" | "bf16" | "fp8"

    def with_tokens(self, t: int) -> "FfnShape":
        return dataclasses.replace(self, tokens=t)


#: The dense layer at the block's decode, prefill and FP8-prefill token counts, and a tiny case
#: for the oracle on every token.
FFN_WORKLOADS = {
    "dense_tiny_fp32": FfnShape("dense_tiny_fp32", tokens=40, dim=256, inter=384, dtype="f32"),
    "dense_decode_bf16": FfnShape("dense_decode_bf16", tokens=16, dim=7168, inter=18432, dtype="bf16"),
    "dense_prefill_bf16": FfnShape("dense_prefill_bf16", tokens=4096, dim=7168, inter=18432, dtype="bf16"),
    "dense_prefill_fp8": FfnShape("dense_prefill_fp8", tokens=16384, dim=7168, inter=18432, dtype="fp8"),
}

_FFN_TID = dict(x=21, w1=22, w3=23, w2=24)


@dataclass
class FfnTensors:
    """Device (or host) tensors of one dense feed-forward workload. Scales are None unless fp8."""

    shape: FfnShape
    x: torch.Tensor
    w1: torch.Tensor
    w3: torch.Tensor
    w2: torch.Tensor
    s1: Optional[torch.Tensor] = None
    s3: Optional[torch.Tensor] = None
    s2: Optional[torch.Tensor] = None


def generate_ffn(shape: FfnShape, seed: int = 0, device="cpu") -> FfnTensors:
    """x ~ N(0, 1) in the activation dtype; w1, w3 [I, D] ~ N(0, 1/D), w2 [D, I] ~ N(0, 1/I), in the
    storage dtype (fp8: e4m3fn codes with one fp32 scale per 128x128 block, as for the experts)."""
    device = torch.device(device)
    t, d, i = shape.tokens, shape.dim, shape.inter
    act = torch.float32 if shape.dtype == "f32" else torch.bfloat16
    x = torch.randn(t, d, generator=_gen(device, seed, _FFN_TID["x"]), device=device, dtype=torch.float32).to(act)
    w1, s1 = _matrix(shape, seed, _FFN_TID["w1"], 0, i, d, d, device)
    w3, s3 = _matrix(shape, seed, _FFN_TID["w3"], 0, i, d, d, device)
    w2, s2 = _matrix(shape, seed, _FFN_TID["w2"], 0, d, i, i, device)
    return FfnTensors(shape, x, w1, w3, w2, s1, s3, s2)

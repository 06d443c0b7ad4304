"""Turn generated torch tensors into the oracle's numpy inputs (exact values)."""
import numpy as np
import torch

from oracle import moe_oracle as O


def exact(t: torch.Tensor) -> np.ndarray:
    """bf16 / fp32 tensor -> float64 numpy array of the same values."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def codes(t: torch.Tensor) -> np.ndarray:
    """float8_e4m3fn tensor -> uint8 codes."""
    return t.detach().to("cpu").contiguous().view(torch.uint8).numpy()


class _Prefetch:
    """expert(e) with the next few experts' fp64 matrices prepared on worker threads (the oracle
    asks for experts in ascending order; the copies and fp8 dequantisations release the GIL).
    Plumbing only: every value comes from `load(e)` unchanged."""

    def __init__(self, load, n_experts, depth=4):
        from concurrent.futures import ThreadPoolExecutor

        self.load, self.n, self.depth = load, n_experts, depth
        self.pool = ThreadPoolExecutor(max_workers=depth)
        self.pending = {}
        self.last_report = -1

    def __call__(self, e):
        for j in range(e, min(self.n, e + self.depth + 1)):
            if j not in self.pending:
                self.pending[j] = self.pool.submit(self.load, j)
        for j in [j for j in self.pending if j < e]:
            self.pending.pop(j).cancel()
        if e // 32 != self.last_report:  # progress of a long oracle run
            self.last_report = e // 32
            print(f"    oracle: expert {e} of {self.n}", flush=True)
        return self.pending.pop(e).result()

    def __del__(self):
        self.pool.shutdown(wait=False, cancel_futures=True)


def expert_fn(tens, prefetch=False):
    """(expert(e), shared()) accessors returning fp64 [out, in] matrices for the oracle; with
    prefetch, the following experts are prepared on worker threads while one is in use."""
    fp8 = tens.shape.dtype == "fp8"

    def mat(w, s):
        if fp8:
            return O.dequant_128x128(codes(w), s.detach().cpu().numpy())
        return exact(w)

    def expert(e):
        if fp8:
            return (mat(tens.w1[e], tens.s1[e]), mat(tens.w3[e], tens.s3[e]), mat(tens.w2[e], tens.s2[e]))
        return exact(tens.w1[e]), exact(tens.w3[e]), exact(tens.w2[e])

    def shared():
        if fp8:
            return mat(tens.ws1, tens.ss1), mat(tens.ws3, tens.ss3), mat(tens.ws2, tens.ss2)
        return exact(tens.ws1), exact(tens.ws3), exact(tens.ws2)

    if prefetch:
        return _Prefetch(expert, tens.shape.n_experts), shared
    return expert, shared


def act_out(shape):
    """(activation storage dtype, output dtype) of a workload."""
    return {"f32": ("f32", "f32"), "bf16": ("bf16", "bf16"), "fp8": ("fp8", "bf16")}[shape.dtype]


def bias_np(tens):
    return None if tens.bias is None else tens.bias.detach().cpu().numpy().astype(np.float32)


def oracle_forward(tens, x=None, prefetch=None):
    """Run the oracle block on tens (optionally on a subset of tokens x [n, D] fp64). Experts are
    prefetched on worker threads for full-size weights (dim >= 4096) unless told otherwise."""
    if prefetch is None:
        prefetch = tens.shape.dim >= 4096
    expert, shared = expert_fn(tens, prefetch=prefetch)
    act, out = act_out(tens.shape)
    xx = exact(tens.x) if x is None else x
    return O.moe_forward(tens.shape, xx, exact(tens.w_gate), bias_np(tens), expert, shared, act, out)


def ffn_mats(tens):
    """fp64 [out, in] weights of a dense feed-forward workload (fp8: dequantised blocks)."""
    if tens.shape.dtype == "fp8":
        return tuple(O.dequant_128x128(codes(w), s.detach().cpu().numpy())
                     for w, s in ((tens.w1, tens.s1), (tens.w3, tens.s3), (tens.w2, tens.s2)))
    return exact(tens.w1), exact(tens.w3), exact(tens.w2)


def oracle_ffn(tens, x=None, mats=None):
    """Run the oracle's dense feed-forward on tens (optionally on tokens x [n, D] fp64)."""
    w1, w3, w2 = ffn_mats(tens) if mats is None else mats
    act, out = act_out(tens.shape)
    return O.dense_ffn(exact(tens.x) if x is None else x, w1, w3, w2, act, out)

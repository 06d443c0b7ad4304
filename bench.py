#!/usr/bin/env python3
"""Throughput of one DeepSeek-V3-style MoE block forward on one MI355X.

A step is one moe_forward (router -> dispatch -> gate/up GEMM + SwiGLU -> down GEMM -> combine)
over one batch of synthetic tokens already resident in HBM. The default workload is the full
block at decode shape: 16 tokens, dim 7168, 256 routed + 1 shared expert (inter 2048), bf16.
The dense_* workloads time instead one moe_ffn, the first layers' dense SwiGLU feed-forward
(dim 7168, inter 18,432), through the same GEMM kernels.

Prints one JSON line: tokens/s, ms per step, the dominant kernel's roofline (algorithmic bytes or
flops per launch over its average duration, from HIP events around that kernel's launches inside
the timed steps) and the CPU oracle timed on a bounded sample of the same workload. A pass of the
same number of untimed steps before the timed ones, with events around every launch, gives the
per-kernel breakdown (`kernels_ms`) and picks the dominant kernel. `step` puts the whole step
against its roofs: algorithmic bytes over the HBM peak and flops over the MFMA peak.

With the default decode headline, `workloads` adds the block's other workloads timed in the same
run (tiny fp32, 4096-token bf16 prefill, skewed 4096-token prefill, 16384-token fp8 prefill), each
with the same step and dominant-kernel figures.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-workloads]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-block tokens/s + % HBM roofline (decode) / % MFMA peak (prefill), 1 GPU"
METRIC_DENSE = "dense-FFN tokens/s + % HBM roofline (decode) / % MFMA peak (prefill), 1 GPU"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="decode_bf16")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-workloads", action="store_true",
                   help="time only the headline workload (by default the decode headline is followed by "
                        "the tiny, prefill, skewed and fp8 workloads)")
    p.add_argument("--side-steps", type=int, default=20, help="timed steps of each further workload")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--calib-copy-mb", type=int, default=0,
                   help="first run a plain device copy of this many MiB (the reference kernel for scaling "
                        "rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes)")
    return p.parse_args()


def kernel_units(shape, counts):
    """Algorithmic bytes and flops per launch of each expert kernel for this routing."""
    D, I, S, T, K = shape.dim, shape.inter, shape.shared_inter, shape.tokens, shape.topk
    wb = 1 if shape.dtype == "fp8" else (4 if shape.dtype == "f32" else 2)
    ab = wb                      # activation storage bytes (x / h)
    ob = 4 if shape.dtype == "f32" else 2
    touched = int((counts > 0).sum())
    R = T * K
    # gate/up: W1 and W3 of every touched expert and the shared expert, x once, h written once
    w13 = touched * 2 * I * D * wb + 2 * S * D * wb
    g1_bytes = w13 + T * D * ab + (R * I + T * S) * ab
    g1_flops = 2 * 2 * D * (R * I + T * S)
    # down: W2 of every touched expert and the shared expert, h read once, expert rows written once
    w2 = touched * I * D * wb + S * D * wb
    g2_bytes = w2 + (R * I + T * S) * ab + (R + T) * D * ob
    g2_flops = 2 * D * (R * I + T * S)
    return touched, {"gemm1": (g1_bytes, g1_flops), "gemm2": (g2_bytes, g2_flops)}


def ffn_units(shape):
    """Algorithmic bytes and flops per launch of the dense feed-forward's two GEMM kernels."""
    D, I, T = shape.dim, shape.inter, shape.tokens
    wb = 1 if shape.dtype == "fp8" else (4 if shape.dtype == "f32" else 2)
    ab, ob = wb, (4 if shape.dtype == "f32" else 2)
    g1 = (2 * I * D * wb + T * D * ab + T * I * ab, 4 * T * D * I)
    g2 = (I * D * wb + T * I * ab + T * D * ob, 2 * T * D * I)
    return {"gemm1": g1, "gemm2": g2}


CSRC = os.path.join(ROOT, "mixture_experts_layer_14_amd", "csrc")


def kernel_base(name):
    """'void moe::gemm_ring_bf16<0, 256>(...)' or '(gemm_ring_bf16<0, RBM>)' -> 'gemm_ring_bf16'."""
    n = name.split("(")[1] if name.startswith("(") else name.split("(")[0]
    n = n.replace("void ", "").replace("moe::", "").strip()
    return n.split("<")[0].strip()


def kernel_key(name):
    """Base name plus the first template argument (the mode), the same for the span names of
    bench.py and the names rocprofv3 prints: '(gemm_ring_bf16<0, RBM>)' -> 'gemm_ring_bf16<0>'."""
    n = name.split("(")[1] if name.startswith("(") else name.split("(")[0]
    n = n.replace("void ", "").replace("moe::", "").strip()
    if "<" not in n:
        return n
    base, rest = n.split("<", 1)
    return f"{base.strip()}<{rest.split(',')[0].split('>')[0].strip()}>"


_INCLUDE = re.compile(r'^\s*#\s*include\s+"([^"]+)"', re.M)


def source_files(kernel):
    """The source file that defines `kernel` and every header of the library it includes,
    directly or through other headers."""
    base = kernel_base(kernel)
    todo = [f for f in sorted(os.listdir(CSRC))
            if f.endswith(".hip") and f"void {base}(" in open(os.path.join(CSRC, f)).read()]
    seen = set()
    while todo:
        f = todo.pop()
        if f in seen or not os.path.exists(os.path.join(CSRC, f)):
            continue
        seen.add(f)
        todo.extend(_INCLUDE.findall(open(os.path.join(CSRC, f)).read()))
    return sorted(seen)


def source_hash(kernel):
    """Hash of the files `kernel` is compiled from (source_files): the counters of a kernel stay
    valid while none of these change."""
    h = hashlib.sha256()
    for f in source_files(kernel):
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, if it was
    taken on the current source of that kernel; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{workload}:{kernel_key(kernel)}")
    if not rec or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(shape, tens, max_tokens, min_seconds=10.0, max_reps=8, dense=False):
    """The oracle as it stands, on the first `max_tokens` tokens of the same inputs, repeated until
    about `min_seconds` of CPU work (at most `max_reps` passes)."""
    from threadpoolctl import threadpool_info

    from tests.oracle_io import exact, ffn_mats, oracle_ffn, oracle_forward

    n = min(max_tokens, shape.tokens)
    x = exact(tens.x[:n])
    mats = ffn_mats(tens) if dense else None
    reps, dt = 0, 0.0
    while reps < max_reps and (reps == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        if dense:
            oracle_ffn(tens, x=x, mats=mats)
        else:
            oracle_forward(tens, x=x, prefetch=False)
        dt += time.perf_counter() - t0
        reps += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": n * reps / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_cores": len(os.sched_getaffinity(0)),
            "sample": f"first {n} of {shape.tokens} tokens of {shape.name}"
                      f"{'' if dense else ', all their experts'}, {reps} pass(es), "
                      f"seconds={dt:.1f}; numpy fp64 with {threads} BLAS threads on a host of "
                      f"{len(os.sched_getaffinity(0))} usable cores"}


def step_units(shape, counts):
    """Algorithmic bytes and flops of one whole forward step (the method's own traffic: every
    touched expert's weights once, the router weight and bias, x and the output) and the time the
    MFMA peak needs for its flops (bf16 or fp32 router, expert GEMMs in the block's dtype)."""
    D, E, K, I, S, T = shape.dim, shape.n_experts, shape.topk, shape.inter, shape.shared_inter, shape.tokens
    wb = 1 if shape.dtype == "fp8" else (4 if shape.dtype == "f32" else 2)
    xb = 4 if shape.dtype == "f32" else 2
    touched = int((counts > 0).sum())
    nbytes = (touched * 3 * I * D + 3 * S * D) * wb + E * D * xb + E * 4 + 2 * T * D * xb
    if shape.dtype == "fp8":  # the fp32 128x128 block scales of the touched weights
        nbytes += (touched * 3 * (I // 128) * (D // 128) + 3 * (S // 128) * (D // 128)) * 4
    router_flops = 2 * T * D * E
    expert_flops = 2 * 3 * D * (T * K * I + T * S)
    peak_router = MFMA_PEAK_TFLOPS["f32" if shape.dtype == "f32" else "bf16"] * 1e12
    t_mfma = router_flops / peak_router + expert_flops / (MFMA_PEAK_TFLOPS[shape.dtype] * 1e12)
    return nbytes, router_flops + expert_flops, t_mfma


def measure(shape, tens, blk, steps, warmup, dense, fused=False):
    """Warm up, time `steps` steps (HIP events around the dominant kernel's launches inside the
    timed region), after an untimed pass of the same length with events around every launch that
    gives the per-kernel breakdown and picks the dominant kernel. fused: each step is one
    moe_forward_fused launch instead of moe_forward."""
    import torch

    from mixture_experts_layer_14_amd import moe

    out = torch.empty_like(tens.x)
    stream = torch.cuda.current_stream()
    if fused:
        plain = blk

        class _Fused:
            ws_view = plain.ws_view

            def forward(self, x, o):
                moe.forward_fused(plain.cfg, plain.wts, x, o, plain.ws)
        blk = _Fused()
    for _ in range(warmup):
        blk.forward(tens.x, out)
    torch.cuda.synchronize()
    T = shape.tokens
    if dense:
        counts, touched, units = None, None, ffn_units(shape)
    else:
        counts = blk.ws_view(T, "counts", torch.int32, shape.n_experts).cpu().numpy()
        touched, units = kernel_units(shape, counts)

    moe.timing_filter(None)
    moe.timing_enable(True)
    for _ in range(steps):
        blk.forward(tens.x, out)
    torch.cuda.synchronize()
    kt = moe.timing_report()
    moe.timing_enable(False)
    kernels = {name: (cnt, tot / cnt) for name, (cnt, tot) in kt.items()}
    dom = max(kernels, key=lambda n: kernels[n][0] * kernels[n][1])

    moe.timing_filter(dom)
    moe.timing_enable(True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        blk.forward(tens.x, out)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    kt_dom = moe.timing_report()
    moe.timing_enable(False)
    moe.timing_filter(None)
    dom_cnt, dom_tot = kt_dom[dom]
    dom_ms = dom_tot / dom_cnt
    kind = "gemm1" if ("gemm1" in dom or "<0" in dom) else ("gemm2" if ("gemm2" in dom or "<1" in dom) else None)
    if fused:  # one kernel is the whole step: its roof is every algorithmic byte of the step
        kind = None
    roof = None
    if kind:
        nbytes, flops = units[kind]
        if T <= 256:
            ach = nbytes / (dom_ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic_from_profiles(dom, shape.name)}
        else:
            peak = MFMA_PEAK_TFLOPS[shape.dtype]
            ach = flops / (dom_ms * 1e-3) / 1e12
            roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(ach / peak, 4), "traffic": traffic_from_profiles(dom, shape.name)}
        roof["kernel"] = dom
        roof["avg_launch_ms"] = round(dom_ms, 5)
    return dict(ms=ms, kernels=kernels, roof=roof, counts=counts, touched=touched)


def block_config(shape, touched, seed):
    return {"workload": shape.name, "tokens": shape.tokens, "dim": shape.dim, "experts": shape.n_experts,
            "groups": shape.n_groups, "topk_groups": shape.topk_groups, "topk": shape.topk,
            "inter": shape.inter, "shared": shape.n_shared, "touched_experts": touched, "seed": seed}


def workload_summary(shape, m):
    """One line of the `workloads` object: the whole step against its binding roof and against
    the MFMA peak, plus the dominant kernel's roofline."""
    nbytes, flops, t_mfma = step_units(shape, m["counts"])
    sec = m["ms"] * 1e-3
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    return {
        "ms_per_step": round(m["ms"], 4), "tokens_per_s": round(shape.tokens / sec, 1),
        "dtype": shape.dtype, "touched_experts": m["touched"],
        "step_bytes": nbytes, "step_flops": flops,
        "hbm_frac": round(t_hbm / sec, 4), "mfma_frac": round(t_mfma / sec, 4),
        "bound": bound, "bound_frac": round(max(t_hbm, t_mfma) / sec, 4),
        "dominant": m["roof"],
        "kernels_ms": {n: round(v[1], 5) for n, v in m["kernels"].items()},
    }


SIDE_WORKLOADS = ["tiny_fp32", "prefill_bf16", "skewed_bf16", "prefill_fp8"]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library has no "
              f"multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch

    from mixture_experts_layer_14_amd import inputs, moe

    dense = args.workload in inputs.FFN_WORKLOADS
    shape = inputs.FFN_WORKLOADS[args.workload] if dense else inputs.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    if args.calib_copy_mb:
        src = torch.ones(args.calib_copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {args.calib_copy_mb} MiB x 3 done", file=sys.stderr, flush=True)
        del src, dst
    print(f"[bench] generating {shape.name} inputs (seed {args.seed})", file=sys.stderr, flush=True)
    if dense:
        tens = inputs.generate_ffn(shape, seed=args.seed, device=dev)
        blk = moe.Ffn(tens, shape.tokens)
    else:
        tens = inputs.generate(shape, seed=args.seed, device=dev)
        blk = moe.Block(tens, shape.tokens)
    print(f"[bench] {shape.name}: {args.steps} steps with per-kernel events, then {args.steps} timed",
          file=sys.stderr, flush=True)
    m = measure(shape, tens, blk, args.steps, args.warmup, dense)
    ms, T = m["ms"], shape.tokens

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(shape, tens, 16, max_reps=400 if dense else 8, dense=dense)

    if dense:
        config = {"workload": shape.name, "tokens": T, "dim": shape.dim, "inter": shape.inter, "seed": args.seed}
    else:
        config = block_config(shape, m["touched"], args.seed)
    rec = {
        "metric": METRIC_DENSE if dense else METRIC, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8", "f32": "f32"}[shape.dtype], "data": "synthetic",
        "config": config,
        "roofline": m["roof"],
        "cpu_baseline": cpu,
        "kernels_ms": {n: round(v[1], 5) for n, v in m["kernels"].items()},
    }
    if not dense:
        rec["step"] = {k: v for k, v in workload_summary(shape, m).items() if k not in ("dominant", "kernels_ms")}

    # The fused single-launch decode on the same inputs (moe_forward_fused), against the headline's
    # separate launches.
    if not dense and not args.no_workloads and args.workload == "decode_bf16":
        print("[bench] decode_bf16: the fused single launch", file=sys.stderr, flush=True)
        mf = measure(shape, tens, blk, args.steps, args.warmup, False, fused=True)
        fs = workload_summary(shape, mf)
        rec["fused_decode"] = {k: fs[k] for k in ("ms_per_step", "tokens_per_s", "hbm_frac", "kernels_ms")}
        rec["fused_decode"]["vs_separate_launches"] = round(ms / mf["ms"], 4)

    # The other workloads of the block, timed in the same run (not the headline value): the tiny
    # fp32 block, the 4096-token bf16 prefill (HBM-bound), the skewed 4096-token prefill and the
    # 16384-token fp8 prefill (MFMA-bound).
    if not args.no_workloads and not dense and args.workload == "decode_bf16":
        del blk, tens
        torch.cuda.empty_cache()
        rec["workloads"] = {}
        for name in SIDE_WORKLOADS:
            sh = inputs.WORKLOADS[name]
            print(f"[bench] {name}: generating inputs", file=sys.stderr, flush=True)
            tw = inputs.generate(sh, seed=args.seed, device=dev)
            bw = moe.Block(tw, sh.tokens)
            steps = max(args.side_steps, 1)
            print(f"[bench] {name}: {steps} steps with per-kernel events, then {steps} timed",
                  file=sys.stderr, flush=True)
            mw = measure(sh, tw, bw, steps, max(args.warmup, 1), False)
            rec["workloads"][name] = workload_summary(sh, mw)
            del bw, tw
            torch.cuda.empty_cache()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

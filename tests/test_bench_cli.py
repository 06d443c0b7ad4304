"""bench.py's host-side contract, without a GPU: the multi-GPU refusal and the helpers that tie
the rocprofv3 traffic summaries to the current kernel sources."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench
from mixture_experts_layer_14_amd import inputs  # noqa: E402


def test_more_than_one_gpu_is_refused_before_touching_a_device():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_names_from_spans_and_from_the_profiler_agree():
    # the bench's span names (macro text) and rocprofv3's demangled names map to the same key
    assert bench.kernel_key("(gemm_ring_bf16<0, RBM, RBN, RBK, RST>)") == "gemm_ring_bf16<0>"
    assert bench.kernel_key("void moe::gemm_ring_bf16<0, 256, 256, 64, 2>(unsigned short const*, int)") == \
        "gemm_ring_bf16<0>"
    assert bench.kernel_key("moe::gemm1_stream_bf16(unsigned short const*, int const*)") == "gemm1_stream_bf16"
    assert bench.kernel_key("gemm1_stream_bf16") == "gemm1_stream_bf16"
    assert bench.kernel_key("void moe::combine<true>(int const*, float const*)") == "combine<true>"
    assert bench.kernel_base("(router_select<1, 1>)") == "router_select"


def test_source_hash_covers_the_defining_file():
    h = bench.source_hash("gemm1_stream_bf16")
    assert h == bench.source_hash("moe::gemm1_stream_bf16(int)")
    assert h != bench.source_hash("combine<true>")  # different defining file


def test_source_files_follow_the_includes():
    """A kernel's counters depend on its own file and the headers it includes, directly or not."""
    ws = bench.source_files("gemm_wstream_bf16<0>")
    assert "gemm_wstream.hip" in ws and "wstream.h" in ws and "kernels.h" in ws
    assert "router_dev.h" not in ws and "router.hip" not in ws
    sel = bench.source_files("router_select<4>")
    assert "router.hip" in sel and "router_dev.h" in sel
    fused = bench.source_files("decode_fused")
    for h in ("router_dev.h", "dispatch_dev.h", "stream_dev.h", "combine_dev.h"):
        assert h in fused


def test_committed_traffic_entries_are_well_formed():
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    recs = json.load(open(path))
    assert recs
    for key, rec in recs.items():
        workload, kernel = key.split(":", 1)
        assert workload in inputs.WORKLOADS or workload in inputs.FFN_WORKLOADS
        assert rec["bytes_per_launch"] > 0
        assert abs(rec["fetch_scale"] - 2.0) < 0.01 and abs(rec["write_scale"] - 1.0) < 0.01
        assert len(rec["source_hash"]) == 16


def test_step_units_match_the_page_figures():
    """Whole-step flops are 796,393,472 per token (every used parameter but the bias, twice); the
    bytes of a step that touches every expert are the block's weights plus x and the output."""
    import numpy as np

    sh = inputs.WORKLOADS["prefill_bf16"]
    nbytes, flops, t_mfma = bench.step_units(sh, np.ones(256, dtype=np.int64))
    assert flops == 4096 * 796_393_472
    assert nbytes == 22_640_329_728 + 2 * 4096 * 7168 * 2
    assert abs(t_mfma - flops / 2.5e15) < 1e-12
    fp8 = inputs.WORKLOADS["prefill_fp8"]
    nb8, fl8, t8 = bench.step_units(fp8, np.ones(256, dtype=np.int64))
    router = 2 * 16384 * 7168 * 256
    assert fl8 == 16384 * 796_393_472 and abs(t8 - (router / 2.5e15 + (fl8 - router) / 5e15)) < 1e-12

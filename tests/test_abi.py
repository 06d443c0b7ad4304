"""The C ABI: libmoe.so loads, exports every function include/moe.h declares, and rejects bad
arguments on the host before any launch (no GPU needed: nothing here reaches a kernel)."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_14_amd import inputs, moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(moe.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    L = moe.lib()
    assert L.moe_status_str(0) == b"ok"
    assert L.moe_status_str(-3) == b"workspace too small"
    assert L.moe_status_str(42) == b"unknown status"


def cfg_of(**kw):
    base = inputs.WORKLOADS["decode_bf16"].replace(**kw)
    return moe.config(base)


def status_of_size(cfg, T=16):
    n = ctypes.c_size_t()
    return moe.lib().moe_workspace_size(ctypes.byref(cfg), T, ctypes.byref(n)), n.value


def test_workspace_size_and_layout():
    st, n = status_of_size(cfg_of(), 16)
    assert st == 0 and n > 0
    st4, n4 = status_of_size(cfg_of(), 4096)
    assert st4 == 0 and n4 > n
    lay = moe.workspace_layout(cfg_of(), 4096)
    assert lay.total == n4
    offs = [lay.idx, lay.w, lay.counts, lay.offsets, lay.row_token, lay.row_of, lay.h_routed, lay.h_shared,
            lay.o_routed, lay.o_shared]
    assert all(o % 256 == 0 for o in offs) and len(set(offs)) == len(offs)
    # o_routed holds T*K rows of dim bf16 values
    assert lay.o_shared - lay.o_routed >= 4096 * 8 * 7168 * 2


@pytest.mark.parametrize("kw,code", [
    (dict(n_groups=7), -2),               # experts not divisible into groups
    (dict(topk_groups=9), -2),            # more kept groups than groups
    (dict(topk=200), -2),                 # topk larger than the kept groups' experts
    (dict(dim=7000), -5),                 # dim not a multiple of 128 for bf16
    (dict(n_experts=2048, n_groups=8), -5),
    (dict(topk=17, topk_groups=8), -5),
    (dict(dim=0), -2),
])
def test_bad_configs_rejected(kw, code):
    st, _ = status_of_size(cfg_of(**kw))
    assert st == code
    assert moe.lib().moe_last_error() != b""


def test_score_func_field():
    """The config's last field selects the router scoring; values other than sigmoid (0) and
    softmax (1) are configuration errors."""
    assert moe.MoeConfig._fields_[-1][0] == "score_func"
    assert status_of_size(cfg_of(score_func="softmax"))[0] == 0
    c = cfg_of()
    c.score_func = 2
    assert status_of_size(c)[0] == -2
    assert b"score_func" in moe.lib().moe_last_error()


def test_negative_tokens_rejected():
    assert status_of_size(cfg_of(), -1)[0] == -1


def test_forward_host_checks_without_gpu():
    L = moe.lib()
    cfg = cfg_of()
    w = moe.MoeWeights(*([0x1000] * 8 + [None] * 6))
    # T = 0 is a no-op
    assert L.moe_forward(ctypes.byref(cfg), ctypes.byref(w), 0x1000, 0, 0x2000, None, 0, None) == 0
    # too small a workspace is caught before anything is launched
    assert L.moe_forward(ctypes.byref(cfg), ctypes.byref(w), 0x1000, 16, 0x2000, 0x3000, 10, None) == -3
    # misaligned pointer
    assert L.moe_forward(ctypes.byref(cfg), ctypes.byref(w), 0x1004, 16, 0x2000, 0x3000, 1 << 40, None) == -1
    # fp8 without scales
    cfg8 = moe.config(inputs.WORKLOADS["prefill_fp8"])
    assert L.moe_forward(ctypes.byref(cfg8), ctypes.byref(w), 0x1000, 16, 0x2000, 0x3000, 1 << 40, None) == -1
    # null weights struct
    assert L.moe_forward(ctypes.byref(cfg), None, 0x1000, 16, 0x2000, 0x3000, 1 << 40, None) == -1


def ffn_size(shape, T):
    n = ctypes.c_size_t()
    cfg = moe.ffn_config(shape)
    return moe.lib().moe_ffn_workspace_size(ctypes.byref(cfg), T, ctypes.byref(n)), n.value


def test_ffn_workspace_size():
    """The dense feed-forward's workspace holds h [T, inter] in the activation dtype (+ x's e4m3 image
    and the scales for fp8), and grows with T; the output is written in place of o_shared."""
    sh = inputs.FFN_WORKLOADS["dense_prefill_bf16"]
    st, n = ffn_size(sh, 4096)
    assert st == 0 and 4096 * 18432 * 2 <= n < 4096 * 18432 * 2 + (1 << 20)
    st16, n16 = ffn_size(sh, 16)
    assert st16 == 0 and n16 < n
    st8, n8 = ffn_size(inputs.FFN_WORKLOADS["dense_prefill_fp8"], 16384)
    assert st8 == 0 and n8 >= 16384 * (18432 + 7168 + (18432 + 7168) // 128 * 4)
    assert ffn_size(sh, 0) == (0, ffn_size(sh, 0)[1])


@pytest.mark.parametrize("dim,inter,dtype,code", [
    (7000, 18432, "bf16", -5),   # dim not a multiple of 128
    (7168, 100, "bf16", -5),     # inter not a multiple of 32
    (7168, 18400, "fp8", -5),    # inter not a multiple of 128 for fp8
    (0, 18432, "bf16", -2),
    (256, 384, "f64", None),     # unknown dtype (checked below)
])
def test_ffn_bad_configs_rejected(dim, inter, dtype, code):
    if dtype == "f64":
        cfg = moe.FfnConfig(256, 384, 7)
        n = ctypes.c_size_t()
        assert moe.lib().moe_ffn_workspace_size(ctypes.byref(cfg), 4, ctypes.byref(n)) == -2
        return
    st, _ = ffn_size(inputs.FfnShape("bad", 4, dim, inter, dtype), 4)
    assert st == code
    assert moe.lib().moe_last_error() != b""


def test_ffn_host_checks_without_gpu():
    L = moe.lib()
    cfg = moe.ffn_config(inputs.FFN_WORKLOADS["dense_decode_bf16"])
    w = moe.FfnWeights(0x1000, 0x1000, 0x1000, None, None, None)
    assert L.moe_ffn(ctypes.byref(cfg), ctypes.byref(w), 0x1000, 0, 0x2000, None, 0, None) == 0   # T = 0
    assert L.moe_ffn(ctypes.byref(cfg), ctypes.byref(w), 0x1000, 16, 0x2000, 0x3000, 10, None) == -3
    assert L.moe_ffn(ctypes.byref(cfg), ctypes.byref(w), 0x1004, 16, 0x2000, 0x3000, 1 << 40, None) == -1
    assert L.moe_ffn(ctypes.byref(cfg), None, 0x1000, 16, 0x2000, 0x3000, 1 << 40, None) == -1
    assert L.moe_ffn(ctypes.byref(cfg), ctypes.byref(w), 0x1000, -1, 0x2000, 0x3000, 1 << 40, None) == -1
    cfg8 = moe.ffn_config(inputs.FFN_WORKLOADS["dense_prefill_fp8"])
    assert L.moe_ffn(ctypes.byref(cfg8), ctypes.byref(w), 0x1000, 16, 0x2000, 0x3000, 1 << 40, None) == -1


def test_static_forward_rejects_tokens_beyond_its_scratch_on_the_host():
    """moe_forward_static refuses, before any device call, a token count whose workspace exceeds
    the library's static array, naming both sizes; T = 0 is a no-op; argument errors come first."""
    L = moe.lib()
    cfg = cfg_of()
    wts = moe.MoeWeights()
    too_many = 1
    while status_of_size(cfg, too_many)[1] <= moe.STATIC_SCRATCH_BYTES:
        too_many *= 2
    st = L.moe_forward_static(ctypes.byref(cfg), ctypes.byref(wts), None, too_many, None, None)
    assert st == -5
    msg = L.moe_last_error().decode()
    assert "static scratch" in msg and str(moe.STATIC_SCRATCH_BYTES) in msg
    assert L.moe_forward_static(ctypes.byref(cfg), ctypes.byref(wts), None, 0, None, None) == 0
    assert L.moe_forward_static(ctypes.byref(cfg), None, None, 0, None, None) == -1
    assert L.moe_forward_static(None, ctypes.byref(wts), None, 4, None, None) == -1
    bad = cfg_of(topk=40)
    assert L.moe_forward_static(ctypes.byref(bad), ctypes.byref(wts), None, 4, None, None) in (-2, -5)
    # the limit in the binding is the header's
    text = open(HEADER).read()
    assert "#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)" in text and moe.STATIC_SCRATCH_BYTES == 64 << 20


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_workspace_size_of_zero_tokens(dtype):
    """T = 0 is valid everywhere: its workspace size is a small positive number (no division by the
    empty token count when the router's k-split is planned)."""
    st, n = status_of_size(cfg_of(dtype=dtype), 0)
    assert st == 0 and 0 < n < 1 << 20
    f = moe.FfnConfig(7168, 18432, {"f32": 0, "bf16": 1, "fp8": 2}[dtype])
    size = ctypes.c_size_t()
    assert moe.lib().moe_ffn_workspace_size(ctypes.byref(f), 0, ctypes.byref(size)) == 0


def test_fused_decode_refuses_other_shapes_on_the_host():
    """moe_forward_fused takes bf16 blocks of 1 to 32 tokens with at most 256 experts; anything else
    is MOE_ERR_UNSUPPORTED before any device call (T = 0 is a no-op)."""
    L = moe.lib()
    wts = moe.MoeWeights()
    n = ctypes.c_size_t(0)
    for cfg, T in [(cfg_of(), 33), (cfg_of(dtype="fp8"), 16), (cfg_of(dtype="f32"), 16),
                   (cfg_of(n_experts=512, n_groups=16), 16)]:
        assert L.moe_forward_fused(ctypes.byref(cfg), ctypes.byref(wts), None, T, None, None, n, None) == -5
        assert "fused decode" in L.moe_last_error().decode()
    assert L.moe_forward_fused(ctypes.byref(cfg_of()), ctypes.byref(wts), None, 0, None, None, n, None) == 0
    assert L.moe_forward_fused(ctypes.byref(cfg_of()), None, None, 4, None, None, n, None) == -1

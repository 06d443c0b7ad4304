"""Pins of the oracle's number formats against library casts and the OCP e4m3fn spec values."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # add exact ties: values halfway between two bf16 neighbours
    base = O.bf16_bits_to_f32(rng.integers(0x3000, 0x4800, 5000).astype(np.uint16))
    ties = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, ties, -ties, np.float32([0.0, -0.0, 1e-40, 3.3e38])])
    ours = O.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(O.bf16_bits_to_f32(ours), torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF only: e4m3fn has no infinities
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_spec_values():
    # OCP OFP8 e4m3fn: bias 7, max normal 448 = 0x7E, min normal 2^-6 = 0x08, min subnormal 2^-9 = 0x01
    assert O.e4m3_decode(np.uint8([0x7E]))[0] == 448.0
    assert O.e4m3_decode(np.uint8([0x08]))[0] == 2.0 ** -6
    assert O.e4m3_decode(np.uint8([0x01]))[0] == 2.0 ** -9
    assert O.e4m3_decode(np.uint8([0x38]))[0] == 1.0
    assert O.e4m3_decode(np.uint8([0xC0]))[0] == -2.0
    # saturation: beyond the largest finite value the code clamps to +-448
    assert list(O.e4m3_encode(np.array([448.0, 460.0, 1e6, -1e6]))) == [0x7E, 0x7E, 0x7E, 0xFE]


def test_e4m3_encode_rne_matches_torch_cast():
    rng = np.random.default_rng(2)
    v = np.concatenate([
        rng.uniform(-448, 448, 100_000),
        rng.standard_normal(100_000) * 0.01,          # subnormal range
        rng.standard_normal(100_000),
    ]).astype(np.float32)
    pos = O.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)  # exact ties (representable in fp32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    v = np.concatenate([v, mids, -mids])
    ours = O.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    same_val = O.e4m3_decode(ours) == O.e4m3_decode(ref)  # +0 and -0 compare equal
    assert same_val.all()


def test_quant_1x128_pins():
    rng = np.random.default_rng(3)
    a = (rng.standard_normal((7, 512)) * rng.uniform(0.01, 10, (7, 1))).astype(np.float32)
    a[3, 128:256] = 0.0                                     # an all-zero block
    q, sc = O.quant_1x128(a)
    assert q.shape == a.shape and sc.shape == (7, 4) and sc.dtype == np.float32
    assert sc[3, 1] == 1.0 and (q[3, 128:256] & 0x7F == 0).all()
    blk = np.abs(a).reshape(7, 4, 128)
    arg = blk.argmax(axis=2)
    for r in range(7):
        for b in range(4):
            if r == 3 and b == 1:
                continue
            assert sc[r, b] == np.float32(blk[r, b].max() / np.float32(448.0))
            assert (q[r, b * 128 + arg[r, b]] & 0x7F) == 0x7E   # the block's amax maps to 448
    # round-to-nearest error bound of a 3-bit mantissa: half an ulp, i.e. 2^-4 relative for normals,
    # and 2^-10 absolute (times the scale) in the subnormal range
    d = O.dequant_1x128(q, sc)
    scale_full = np.repeat(sc, 128, axis=1).astype(np.float64)
    err = np.abs(d - a.astype(np.float64)) / scale_full
    mag = np.abs(a.astype(np.float64)) / scale_full
    assert (err <= np.maximum(mag * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)).all()


def test_dequant_128x128_is_blockwise():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 0x7E, (256, 384)).astype(np.uint8)
    sc = rng.uniform(0.5, 2.0, (2, 3)).astype(np.float32)
    d = O.dequant_128x128(codes, sc)
    sc2 = sc.copy()
    sc2[1, 2] *= 2
    d2 = O.dequant_128x128(codes, sc2)
    changed = d2 != d
    assert changed[128:, 256:].sum() == (d[128:, 256:] != 0).sum() and not changed[:128].any()
    assert not changed[:, :256].any()
    assert np.array_equal(d2[128:, 256:], 2 * d[128:, 256:])


@pytest.mark.parametrize("n", [1, 5])
def test_quant_sign_and_zero(n):
    a = np.zeros((n, 128), np.float32)
    a[:, 0] = -3.0
    q, sc = O.quant_1x128(a)
    assert (q[:, 0] == 0xFE).all() and np.allclose(sc, 3.0 / 448.0)

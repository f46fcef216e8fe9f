"""Pins for the FP8 (E4M3, block-scaled) oracle: decode against the format's definition and
hand values, the quantizer against torch's own float8_e4m3fn conversion and brute force, the
block exponent against its defining inequality, and planted mistakes."""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as f8


def test_e4m3_hand_values():
    # sign, 4-bit exponent (bias 7), 3-bit mantissa; exponent 0 is subnormal (m/8 * 2^-6)
    codes = [0x00, 0x01, 0x07, 0x08, 0x38, 0x39, 0x3F, 0x40, 0x77, 0x7E, 0x80, 0xB8, 0xFE]
    want = [0.0, 2 ** -9, 7 * 2 ** -9, 2 ** -6, 1.0, 1.125, 1.875, 2.0, 240.0, 448.0, -0.0, -1.0,
            -448.0]
    np.testing.assert_array_equal(f8.e4m3_value(codes), want)
    assert np.isnan(f8.e4m3_value([0x7F, 0xFF])).all()


def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = f8.e4m3_value(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


def _torch_codes(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_quantize_matches_torch_conversion():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 2.0 ** rng.integers(-14, 8, 20000),
        # exact midpoints between neighbouring codes (ties) and the codes themselves
        (f8._POS_VALUES[1:] + f8._POS_VALUES[:-1]) / 2, -(f8._POS_VALUES[1:] + f8._POS_VALUES[:-1]) / 2,
        f8._POS_VALUES, [0.0, -0.0, 448.0, -448.0, 2 ** -10, 3 * 2 ** -11],
    ])
    np.testing.assert_array_equal(f8.quantize_e4m3(x), _torch_codes(x))


def test_quantize_is_nearest_by_brute_force():
    rng = np.random.default_rng(1)
    x = rng.uniform(-448, 448, 3000)
    codes = f8.quantize_e4m3(x)
    allv = f8.e4m3_value(np.arange(256))
    finite = ~np.isnan(allv)
    best = np.min(np.abs(x[:, None] - allv[None, finite]), axis=1)
    np.testing.assert_array_equal(np.abs(x - f8.e4m3_value(codes)), best)
    assert np.all(f8.quantize_e4m3([500.0, -1e9]) == [0x7E, 0xFE])   # saturation


def test_block_exponent_is_the_largest_that_fits():
    rng = np.random.default_rng(2)
    amax = np.concatenate([rng.uniform(0, 1, 2000) * 2.0 ** rng.integers(-130, 126, 2000),
                           [448.0, 448.0 * 2 ** -5, 449.0, 2 ** -140, 1e30]])
    amax = amax[amax > 0]
    e = f8.block_exponent(amax)
    fits = amax * np.ldexp(1.0, e) <= 448
    assert fits.all()
    nxt = amax * np.ldexp(1.0, e + 1) > 448
    assert np.all(nxt | (e == 127))
    assert f8.block_exponent(np.array([0.0]))[0] == 0


def test_mxfp8_roundtrip_error_bound():
    # three mantissa bits: each element is within half a unit of its block's grid
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 5, 128)) * 2.0 ** rng.integers(-8, 8, (7, 5, 1))
    codes, scales = f8.quantize_mxfp8(x)
    assert codes.dtype == np.uint8 and scales.shape == (7, 5, 4)
    xd = f8.dequantize_mxfp8(codes, scales)
    step = np.ldexp(1.0, scales.astype(np.int64) - 127)    # 2^-e of each block
    xb, db = x.reshape(7, 5, 4, 32), xd.reshape(7, 5, 4, 32)
    err = np.abs(xb - db)
    bound = np.maximum(np.abs(xb) * 2.0 ** -4, 2.0 ** -10 * step[..., None])
    assert np.all(err <= bound * (1 + 1e-12))
    # the block maximum lands in the top binade: amax * 2^e in (224, 448]
    top = np.max(np.abs(xb), axis=-1) / step
    assert np.all((top > 224) & (top <= 448))


def test_mxfp8_exact_for_representable_blocks():
    # values already on a block's E4M3 grid survive unchanged, and attention on them is exact
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 0x7F, (1, 2, 9, 64)).astype(np.uint8) | (rng.integers(0, 2, (1, 2, 9, 64)) * 0x80).astype(np.uint8)
    codes[..., ::32] = 0x7E   # every block holds 448, so its exponent is 0
    x = f8.e4m3_value(codes) * 2.0 ** -6
    c2, s2 = f8.quantize_mxfp8(x)
    np.testing.assert_array_equal(f8.dequantize_mxfp8(c2, s2), x)
    v = np.random.default_rng(5).standard_normal((1, 2, 9, 64))
    o1, l1 = f8.attention_forward_fp8qk(x, x, v, 0.05, True)
    o2, l2 = oracle.attention_forward(x, x, v, 0.05, True)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


def test_fp8qk_close_to_exact_attention():
    # the quantization error of S stays small for unit-normal inputs at D = 128
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((1, 2, 200, 128)) for _ in range(3))
    o1, l1 = f8.attention_forward_fp8qk(q, k, v, 1 / math.sqrt(128), True)
    o2, l2 = oracle.attention_forward(q, k, v, 1 / math.sqrt(128), True)
    assert np.max(np.abs(l1 - l2)) < 0.1 and np.max(np.abs(o1 - o2)) < 0.15


def _quant_pins_pass():
    try:
        test_quantize_matches_torch_conversion()
        test_block_exponent_is_the_largest_that_fits()
        test_mxfp8_roundtrip_error_bound()
    except AssertionError:
        return False
    return True


def test_planted_quantizer_mistakes_are_caught(monkeypatch):
    real_q, real_e = f8.quantize_e4m3, f8.block_exponent

    def ties_away(x):   # round half away from zero instead of to even
        x = np.asarray(x, dtype=np.float64)
        c = real_q(x)
        v = f8.e4m3_value(c)
        up = real_q(np.nextafter(np.abs(x), np.inf)) | np.where(x < 0, 0x80, 0).astype(np.uint8)
        tie = np.abs(np.abs(x) - np.abs(v)) > 0
        return np.where(tie & (np.abs(f8.e4m3_value(up)) > np.abs(v)), up, c).astype(np.uint8)

    def exponent_one_high(amax):
        return real_e(amax) + 1

    for name, wrong in (("quantize_e4m3", ties_away), ("block_exponent", exponent_one_high)):
        monkeypatch.setattr(f8, name, wrong)
        assert not _quant_pins_pass(), name
        monkeypatch.setattr(f8, name, real_q if name == "quantize_e4m3" else real_e)
    assert _quant_pins_pass()

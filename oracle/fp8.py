"""CPU oracle for the FP8 (E4M3) Q K^T variant of exact attention: test infrastructure only.

Nothing in the product path may import, call or link this module; only the tests, the smoke
check and the CPU-baseline leg of the benchmark use it. It shares no code with the HIP path.

Source: "Lab 06 - Attention kernels", "Stretch" list (FP8 E4M3 Q and K for the Q K^T product,
accuracy measured against speed). The pages fix neither the FP8 encoding details nor the
scaling, so this module takes the plainest readings and states them:

  * E4M3 is the OCP 8-bit format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 encodes subnormals m/8 * 2^-6; there is no infinity, and the two codes
    with every exponent and mantissa bit set are NaN. The largest finite magnitude is 448.
  * Rounding is to the nearest E4M3 value, ties to the code with an even mantissa (the usual
    IEEE rule); magnitudes above 448 saturate to 448.
  * Scaling is per block of 32 consecutive elements along the head dimension, by a power of
    two: the block exponent e is the largest integer with amax * 2^e <= 448 (amax the block's
    largest magnitude), clamped to e <= 127; an all-zero block takes e = 0. The scale is stored
    as the byte 127 - e (an E8M0 exponent: the block's values are code values times
    2^(byte - 127)). A power of two keeps the scaling exact, so the codes are a function of the
    inputs alone, not of any rounding in the scaling.
  * Only Q and K are quantized; V, P and the P V product stay as in the bf16 forward.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_forward_gqa

BLOCK = 32
E4M3_MAX = 448.0


def e4m3_value(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8) as float64; NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    mag = np.where(ex == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * 2.0 ** (ex - 7))
    mag = np.where((ex == 15) & (man == 7), np.nan, mag)
    return sign * mag


# the 127 non-negative finite codes in increasing value order (code 0x00 .. 0x7E)
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = e4m3_value(_POS_CODES)


def quantize_e4m3(x) -> np.ndarray:
    """Nearest E4M3 code to each value of x (float64), ties to the even code, saturating at
    448; the sign bit follows x's (so -0.0 and small negatives that round to zero give 0x80).
    x must hold no NaN."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("quantize_e4m3: NaN input")
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(a == 0, 0, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def block_exponent(amax) -> np.ndarray:
    """Largest integer e with amax * 2^e <= 448 (amax > 0), clamped to e <= 127; 0 where
    amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    e = np.floor(np.log2(E4M3_MAX / safe)).astype(np.int64)
    # correct the floor of the logarithm by exact power-of-two checks
    e = np.where(safe * np.ldexp(1.0, e + 1) <= E4M3_MAX, e + 1, e)
    e = np.where(safe * np.ldexp(1.0, e) > E4M3_MAX, e - 1, e)
    e = np.minimum(e, 127)
    return np.where(amax > 0, e, 0)


def quantize_mxfp8(x):
    """Block-scaled E4M3 of x (..., D), D a multiple of 32: returns (codes uint8 (..., D),
    scale bytes uint8 (..., D / 32)), scale byte = 127 - e per block."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if D % BLOCK:
        raise ValueError("the last axis must be a multiple of 32")
    xb = x.reshape(x.shape[:-1] + (D // BLOCK, BLOCK))
    e = block_exponent(np.max(np.abs(xb), axis=-1))
    codes = quantize_e4m3(xb * np.ldexp(1.0, e)[..., None])
    return codes.reshape(x.shape), (127 - e).astype(np.uint8)


def dequantize_mxfp8(codes, scales) -> np.ndarray:
    """Values of block-scaled E4M3 data: code value times 2^(scale byte - 127)."""
    v = e4m3_value(codes)
    D = v.shape[-1]
    vb = v.reshape(v.shape[:-1] + (D // BLOCK, BLOCK))
    s = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return (vb * s[..., None]).reshape(v.shape)


def attention_forward_fp8qk(q, k, v, scale: float, causal: bool):
    """Exact attention (float64, as `attention_forward_gqa`) on Q and K replaced by their
    block-scaled E4M3 values: what an FP8 Q K^T path computes up to summation order.
    q (B, Hq, Tq, D), k and v (B, Hkv, Tk, D) float64."""
    qd = dequantize_mxfp8(*quantize_mxfp8(q))
    kd = dequantize_mxfp8(*quantize_mxfp8(k))
    return attention_forward_gqa(qd, kd, np.asarray(v, dtype=np.float64), scale, causal)

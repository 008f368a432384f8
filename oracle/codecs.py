"""Number formats used by the oracle: bfloat16 rounding, OCP FP8 E4M3, int8.

TEST INFRASTRUCTURE ONLY (see the package header).

Why these formats: the TRTLLM Attention page (section "SAGE quantization")
and the Diffusion Attention Backends page (section "TRTLLM_ATTN SAGE
Quantization") quantize Q and K to int8 or fp8_e4m3 and V to fp8_e4m3; the
dense path is BF16 (TRTLLM Attention, section "Dense mode").  The pages give
neither the rounding rule nor the saturation rule; the readings taken here
are round-to-nearest-even everywhere and saturation to the largest finite
code (OCP "satfinite"), with E4M3 being the OCP OFP8 E4M3 format (bias 7,
3 mantissa bits, subnormals m * 2**-9, no infinities, 0x7F/0xFF = NaN,
largest finite 448).

Parity pins (tests/test_oracle_codecs.py): decode against torch's
float8_e4m3fn for all 256 codes; encode against torch's float8_e4m3fn
conversion in range; saturation beyond 448 against the closed form;
bf16 rounding against torch's bfloat16 conversion; int8 rounding against
numpy's rint.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
INT8_MAX = 127.0
_BF16_MAX = float.fromhex("0x1.fep127")


def f32(x):
    """Round to IEEE binary32, nearest-even (numpy's float64 -> float32 cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_round(x):
    """Round float64 values straight to bfloat16 (RNE), returned as float64.

    Works from the float64 value itself (no detour through binary32, whose
    double rounding is not innocuous for arbitrary float64 inputs).
    bfloat16 has 8 significant bits and binary32's exponent range.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)
    ex = np.maximum(e - 1, -126)            # binade exponent, floored at the normal minimum
    quantum = np.ldexp(1.0, ex - 7)
    with np.errstate(invalid="ignore", over="ignore"):
        val = np.rint(a / quantum) * quantum
    val = np.where(val > _BF16_MAX, np.inf, val)
    val = np.where(np.isnan(a), np.nan, val)
    return np.copysign(val, x)


_CHUNK = 1 << 16


def _elementwise(fn, x, out_dtype, in_dtype=np.float64):
    """Apply the elementwise ``fn`` to ``x`` in slices of 64K elements (the
    same values as one call; small slices stay in cache, which makes large
    tensors an order of magnitude faster)."""
    x = np.asarray(x, dtype=in_dtype)
    if x.size <= _CHUNK:
        return fn(x)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, out_dtype)
    for i in range(0, flat.size, _CHUNK):
        out[i:i + _CHUNK] = fn(flat[i:i + _CHUNK])
    return out.reshape(x.shape)


def e4m3_encode(x):
    """OCP E4M3 code (uint8) of each value: RNE, satfinite, sign kept.

    The value is rounded on the E4M3 grid of its binade (quantum 2**(e-3) for
    binade 2**e, e >= -6; the subnormal quantum 2**-9 below that), then
    clamped to 448.  -0 encodes as 0x80.  NaN encodes as 0x7F (| sign).
    """
    return _elementwise(_e4m3_encode, x, np.uint8)


def _e4m3_encode(x):
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    _, e = np.frexp(a)
    ex = np.maximum(e - 1, -6)
    quantum = np.ldexp(1.0, ex - 3)
    with np.errstate(invalid="ignore", over="ignore"):
        n = np.rint(a / quantum)
    val = np.minimum(n * quantum, E4M3_MAX)
    # encode the rounded magnitude
    sub = val < 2.0 ** -6
    code_sub = np.rint(val * 2.0 ** 9)                      # 0..8 (8 == smallest normal)
    _, e2 = np.frexp(np.where(sub, 1.0, val))
    biased = (e2 - 1) + 7
    mant = np.rint((np.where(sub, 1.0, val) / np.ldexp(1.0, e2 - 1) - 1.0) * 8.0)
    code_norm = biased * 8 + mant
    code = np.where(sub, code_sub, code_norm).astype(np.int64)
    code = np.where(nan, 0x7F, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def e4m3_decode(code):
    """Value (float64) of each OCP E4M3 code; 0x7F and 0xFF decode to NaN."""
    return _elementwise(_e4m3_decode, code, np.float64, np.int64)


def _e4m3_decode(code):
    c = np.asarray(code, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(ef == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, ef - 7))
    val = np.where((ef == 15) & (m == 7), np.nan, val)
    return sign * val


def int8_code(x):
    """Symmetric int8 code: round half to even, clamp to [-127, 127]."""
    r = np.rint(np.asarray(x, dtype=np.float64))
    return np.clip(r, -INT8_MAX, INT8_MAX).astype(np.int8)

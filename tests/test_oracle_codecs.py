"""Pins of the oracle's number formats against torch's own conversions,
the OCP OFP8 specification's listed values, and closed forms."""
import math

import numpy as np
import pytest
import torch

from oracle import bf16_round, e4m3_decode, e4m3_encode, int8_code

GOLDEN = __file__.rsplit("/", 1)[0] + "/golden/e4m3_ocp_reference_values.txt"


def _torch_e4m3_codes(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_decode_matches_ocp_listed_values():
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = float(e4m3_decode(np.array([int(code, 16)]))[0])
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_encode_decode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert len(codes) == 254
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    mags = np.exp2(rng.uniform(-14, math.log2(448.0), 2_000_000)).astype(np.float32)
    x = np.where(rng.random(mags.shape) < 0.5, -mags, mags).astype(np.float32)
    # every midpoint between neighbouring finite codes, and the floats right beside them
    vals = np.unique(e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    x = np.concatenate([x, near, -near, vals.astype(np.float32), np.float32([0.0, -0.0, 448.0, -448.0])])
    x = x[np.abs(x) <= 448.0]
    assert np.array_equal(e4m3_encode(x), _torch_e4m3_codes(x))


def test_encode_saturates_beyond_448():
    x = np.array([448.5, 463.9, 464.0, 1e4, 3e38, np.inf], dtype=np.float64)
    assert np.all(e4m3_encode(x) == 0x7E)
    assert np.all(e4m3_encode(-x) == 0xFE)
    # below 464 torch agrees (round to nearest even on the 448 grid point)
    y = np.float32([448.5, 463.9])
    assert np.array_equal(e4m3_encode(y), _torch_e4m3_codes(y))


def test_encode_nan_and_signed_zero():
    assert e4m3_encode(np.array([np.nan]))[0] & 0x7F == 0x7F
    assert e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert e4m3_encode(np.array([0.0]))[0] == 0x00


def test_bf16_round_matches_torch_for_binary32_inputs():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(1_000_000) * np.exp2(rng.uniform(-130, 120, 1_000_000))).astype(np.float32)
    bits = rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    bits = bits[np.isfinite(bits)]
    x = np.concatenate([x, bits])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_is_single_rounding_from_float64():
    # 1 + 2**-8 + 2**-30 lies above the bf16 midpoint 1 + 2**-8; rounding via
    # binary32 first would land on the midpoint and then round to even (1.0).
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert bf16_round(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0            # exact tie -> even
    assert bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert bf16_round(np.array([float.fromhex("0x1.ffp127")]))[0] == math.inf


@pytest.mark.parametrize("x,c", [(0.5, 0), (1.5, 2), (2.5, 2), (-2.5, -2), (-0.5, 0),
                                 (126.5, 126), (127.4, 127), (127.6, 127), (300.0, 127),
                                 (-127.6, -127), (-1e9, -127)])
def test_int8_code_half_even_and_clamp(x, c):
    assert int(int8_code(np.array([x]))[0]) == c

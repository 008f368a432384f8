"""Pins of the oracle's QK16PV8 and MXFP8 recipes: the MX block quantizer
(scalar brute force, power-of-two scales, saturation, error bounds), the
tensor-wide V scale, and equality of the attention emulation with exact
attention where every quantization step is exact."""
import math

import numpy as np
import pytest
import torch

from oracle import E4M3_MAX, e4m3_decode, e4m3_encode, exact_attention, sage_attention, sage_quantize, \
    sage_skip_attention
from oracle.attention import _mx_quant_rows
from diffusion_transformer_attention_non_amd.synth import gaussian_qkv

SC = 1 / math.sqrt(128)
E4M3_VALUES = np.unique(np.abs(e4m3_decode(np.arange(256, dtype=np.uint8))))
E4M3_VALUES = E4M3_VALUES[np.isfinite(E4M3_VALUES)]


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)


def _scalar_mx_block(vals):
    """One 32-element block by the MX definition, with Python scalars."""
    amax = max(abs(float(x)) for x in vals)
    if amax == 0.0:
        e = -127
    else:
        m, ex = math.frexp(amax)                 # amax = m * 2**ex, 0.5 <= m < 1
        e = min(127, max(-127, (ex - 1) - 8))    # floor(log2 amax) - emax(E4M3)
    codes = [int(e4m3_encode(np.float64(float(x) / 2.0 ** e))) for x in vals]
    return codes, e


def test_mx_quantizer_matches_scalar_definition():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((5, 128)) * np.exp(rng.uniform(-8, 8, (5, 1)))).astype(np.float32)
    x[2, 32:64] = 0.0                                   # an all-zero block
    x[3, :32] = 448.0 * 2.0 ** -3                       # amax exactly at the top of a binade
    codes, exps = _mx_quant_rows(x)
    for r in range(5):
        for b in range(4):
            c, e = _scalar_mx_block(x[r, 32 * b:32 * b + 32])
            assert exps[r, b] == e
            assert list(codes[r, 32 * b:32 * b + 32]) == c


def test_mx_scale_exponents_and_saturation():
    x = np.zeros((4, 128), np.float32)
    x[0, :32] = 1.0                        # floor(log2 1) - 8 = -8: codes 256 = 1.0 * 2**8
    x[1, :32] = 448.0                      # X = 1: E4M3 values pass through unchanged
    x[2, :32] = 0.75                       # floor(log2 0.75) = -1 -> X = 2**-9, 0.75 * 512 = 384
    x[3, :32] = 500.0                      # 500 / 2**0 = 500 saturates to 448
    codes, exps = _mx_quant_rows(x)
    assert list(exps[:, 0]) == [-8, 0, -9, 0]
    dec = e4m3_decode(codes[:, 0])
    assert list(dec) == [256.0, 448.0, 384.0, 448.0]
    assert (exps[:, 1:] == -127).all() and not codes[:, 32:].any()


def test_mx_roundtrip_error_bound():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((64, 128)) * 3).astype(np.float32)
    codes, exps = _mx_quant_rows(x)
    X = np.repeat(np.ldexp(1.0, exps), 32, axis=1)
    dec = e4m3_decode(codes) * X
    ratio = np.abs(x) / X
    normal = (ratio >= 2.0 ** -6) & (ratio <= E4M3_MAX)
    sat = ratio > E4M3_MAX
    # RNE on a 3-bit mantissa: relative error <= 2**-4 in the normal range,
    # absolute <= 2**-10 X below it; above 448 X the value saturates to 448 X
    assert np.all(np.abs(dec - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal] * (1 + 1e-12))
    sub = ratio < 2.0 ** -6
    assert np.all(np.abs(dec - x)[sub] <= 2.0 ** -10 * X[sub] * (1 + 1e-12))
    assert np.all(np.abs(dec[sat]) == E4M3_MAX * X[sat])
    assert sat.any()
    blk = ratio.reshape(64, 4, 32).max(axis=2)
    assert np.all((blk >= 256) & (blk < 512))


def test_tensor_wide_v_scale():
    rng = np.random.default_rng(3)
    q = _bf16(rng.standard_normal((2, 40, 2, 128)))
    k = _bf16(rng.standard_normal((2, 40, 2, 128)))
    v = _bf16(rng.standard_normal((2, 40, 2, 128)) * 3)
    quant = sage_quantize(q, k, v, "bf16", 0, 0, 0)
    vmax = float(v.float().abs().max())
    assert np.all(quant["v_scale"] == np.float32(np.float32(vmax) / np.float32(E4M3_MAX)))
    assert (np.abs(e4m3_decode(quant["v_codes"])).max()) == E4M3_MAX
    assert not quant["mu"].any()                      # no smoothing outside SageAttention
    np.testing.assert_array_equal(quant["q_codes"], q.float().numpy().transpose(0, 2, 1, 3))


def _exact_v(rng, shape):
    """V whose E4M3 quantization is exact with a tensor-wide or a per-channel
    scale: E4M3 values times 2**-5, with 448 in every (head, channel)."""
    c = rng.choice(E4M3_VALUES, size=shape) * rng.choice([-1.0, 1.0], size=shape)
    c[:, 0] = E4M3_MAX
    return c * 2.0 ** -5


def test_qk16pv8_equals_exact_attention_without_p_rounding():
    rng = np.random.default_rng(4)
    q = _bf16(rng.standard_normal((1, 70, 4, 128)))
    k = _bf16(rng.standard_normal((1, 70, 2, 128)))
    v = _bf16(_exact_v(rng, (1, 70, 2, 128)))
    quant = sage_quantize(q, k, v, "bf16", 0, 0, 0)
    got = sage_attention(quant, SC, 64, quantize_p=False)
    ref = exact_attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), SC)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def _exact_mx(rng, shape):
    """Rows whose MX quantization is exact: per 32-block E4M3 values times
    2**e with the block's largest code in [256, 448]."""
    S, H, D = shape[1], shape[2], shape[3]
    x = np.empty(shape)
    for s in range(S):
        for h in range(H):
            for b in range(D // 32):
                c = rng.choice(E4M3_VALUES[E4M3_VALUES <= 448], 32) * rng.choice([-1.0, 1.0], 32)
                c[rng.integers(32)] = rng.choice(E4M3_VALUES[(E4M3_VALUES >= 256)])
                x[0, s, h, 32 * b:32 * b + 32] = c * 2.0 ** int(rng.integers(-14, -6))
    return x


@pytest.mark.parametrize("vb", [0, 1])
def test_mxfp8_equals_exact_attention_on_exact_inputs(vb):
    rng = np.random.default_rng(5 + vb)
    q = _bf16(_exact_mx(rng, (1, 40, 2, 128)))
    k = _bf16(_exact_mx(rng, (1, 40, 1, 128)))
    v = _bf16(_exact_v(rng, (1, 40, 1, 128)))
    assert np.array_equal(q.double().numpy(), _exact_mx(np.random.default_rng(5 + vb), (1, 40, 2, 128)))
    quant = sage_quantize(q, k, v, "mxfp8", 0, 0, vb)
    got = sage_attention(quant, SC, 64, quantize_p=False)
    ref = exact_attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), SC)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_mxfp8_and_qk16pv8_close_to_exact_with_p_rounding():
    rng = np.random.default_rng(7)
    q = _bf16(rng.standard_normal((1, 200, 2, 128)))
    k = _bf16(rng.standard_normal((1, 200, 2, 128)))
    v = _bf16(rng.standard_normal((1, 200, 2, 128)))
    ref = exact_attention(q, k, v, SC)
    for rec in (("bf16", 0, 0, 0), ("mxfp8", 0, 0, 0), ("mxfp8", 0, 0, 1)):
        got = sage_attention(sage_quantize(q, k, v, *rec), SC, 64)
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert rel < 0.06, (rec, rel)


def test_recipe_blocks_validated():
    q = _bf16(np.ones((1, 4, 1, 128)))
    for rec in (("bf16", 1, 1, 1), ("bf16", 0, 0, 1), ("mxfp8", 0, 0, 2), ("mxfp8", 1, 0, 0), ("int8", 1, 16, 0),
                ("nvfp4", 0, 0, 0)):
        with pytest.raises(ValueError):
            sage_quantize(q, q, q, *rec)


def test_skip_on_mxfp8_reduces_to_sage_at_factor_zero():
    rng = np.random.default_rng(8)
    q = _bf16(rng.standard_normal((1, 96, 1, 128)) * 2)
    k = _bf16(rng.standard_normal((1, 96, 1, 128)) * 2)
    v = _bf16(rng.standard_normal((1, 96, 1, 128)))
    quant = sage_quantize(q, k, v, "mxfp8", 0, 0, 1)
    o, sk, _, rows = sage_skip_attention(quant, SC, 0.0, 32, 64)
    assert not sk.any() and np.array_equal(o, sage_attention(quant, SC, 64, rows=rows))


def test_tensor_wide_v_scale_from_a_slice():
    """v_amax: quantizing one head with the tensor-wide maximum gives that head's part of
    the whole-tensor quantization ("Recipes": one V scale for the whole tensor)."""
    q, k, v = gaussian_qkv(1, 40, 2, 2, seed=5)
    full = sage_quantize(q, k, v, "bf16", 0, 0, 0)
    amax = float(np.abs(v.float().numpy()).max())
    for h in range(2):
        part = sage_quantize(q[:, :, h:h + 1], k[:, :, h:h + 1], v[:, :, h:h + 1], "bf16", 0, 0, 0, v_amax=amax)
        assert np.array_equal(part["v_codes"][:, 0], full["v_codes"][:, h])
        assert np.array_equal(part["v_scale"][:, 0], full["v_scale"][:, h])
    with pytest.raises(ValueError):
        sage_quantize(q, k, v, "bf16", 0, 0, 0, v_amax=amax / 2)


@pytest.mark.parametrize("order,block_n", [((0, 1), 2), ((0, 1), 1), ((1, 0), 1)])
def test_p_rounding_closed_forms(order, block_n):
    """Two keys with logits s = 0.9 ln 2 ("hot") and 0 ("cold"); V = 1 on the hot key in
    channel 0 and on the cold key in channel 1; c = 2^-0.9.  Against the running maximum
    0.9 ln 2, p = (1, c), and 2^8 c = 137.19 rounds to the E4M3 value 144 (between 128 and
    144); the row sum adds the unrounded p.  So with both keys in one tile, or the hot key
    first, O = (1, 144/256) / (1 + c).  With the cold key first its p was rounded at p = 1
    (exact) and the later rescale by c is exact in float64: O = (1, c) / (1 + c).  A dropped
    2^8, a row sum of the rounded p, a reference rounded up to a power of two, or a floor
    reference would each give other values.  Without P rounding: exact softmax."""
    q = torch.zeros(1, 1, 1, 128)
    k = torch.zeros(1, 2, 1, 128)
    v = torch.zeros(1, 2, 1, 128)
    q[0, 0, 0, 0] = 1.0
    hot, cold = order
    k[0, hot, 0, 0] = 1.0
    v[0, hot, 0, 0] = 1.0
    v[0, cold, 0, 1] = 1.0
    sm = 0.9 * math.log(2.0)
    quant = sage_quantize(q.bfloat16(), k.bfloat16(), v.bfloat16(), "bf16", 0, 0, 0)
    v1 = 448.0 * float(np.float32(1.0 / 448.0))   # V = 1 dequantized: code 448 times binary32(1 / 448)
    c = 2.0 ** -0.9
    o = sage_attention(quant, sm, block_n)
    cold_p = c if order == (1, 0) and block_n == 1 else 144.0 / 256.0
    assert abs(o[0, 0, 0, 0] - v1 / (1 + c)) < 1e-12
    assert abs(o[0, 0, 0, 1] - cold_p * v1 / (1 + c)) < 1e-12
    assert np.all(o[0, 0, 0, 2:] == 0.0)
    o_exact = sage_attention(quant, sm, block_n, quantize_p=False)
    assert abs(o_exact[0, 0, 0, 0] - 2 ** 0.9 / (2 ** 0.9 + 1) * v1) < 1e-12
    assert abs(o_exact[0, 0, 0, 1] - 1 / (2 ** 0.9 + 1) * v1) < 1e-12

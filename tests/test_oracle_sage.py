"""Pins of the oracle's SAGE quantizer and SAGE attention emulation:
closed forms, error bounds, brute force on tiny inputs, and equality with
exact attention where every quantization step is exact."""
import math
import struct

import numpy as np
import pytest
import torch

from oracle import (E4M3_MAX, INT8_MAX, e4m3_decode, exact_attention, k_channel_mean,
                    sage_attention, sage_quantize)

U32 = 2.0 ** -24


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)


def _gauss_inputs(B, S, Hq, Hkv, seed, bias_std=4.0, outliers=4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, S, Hq, 128)).astype(np.float32)
    k = rng.standard_normal((B, S, Hkv, 128)).astype(np.float32)
    v = rng.standard_normal((B, S, Hkv, 128)).astype(np.float32)
    bias = rng.standard_normal((Hkv, 128)).astype(np.float32) * bias_std
    bias[:, rng.choice(128, outliers, replace=False)] *= 8
    k += bias
    return _bf16(q), _bf16(k), _bf16(v)


def _dec(c, dt):
    return c.astype(np.float64) if dt == "int8" else e4m3_decode(c)


# ---------------------------------------------------------------- K mean

def test_k_mean_matches_scalar_float32_loop():
    rng = np.random.default_rng(3)
    k = _bf16(rng.standard_normal((1, 600, 2, 128)) * 3 + 5).float().numpy()
    mu = k_channel_mean(k)
    for g in range(2):
        for d in (0, 1, 77, 127):
            tot = np.float32(0.0)
            for c0 in range(0, 600, 256):
                acc = np.float32(0.0)
                for s in range(c0, min(600, c0 + 256)):
                    acc = np.float32(acc + k[0, s, g, d])
                tot = np.float32(tot + acc)
            assert np.float32(tot / np.float32(600)) == mu[0, g, d]


def test_k_mean_chunked_order_differs_from_flat_order():
    k = np.ones((1, 512, 1, 128), np.float32)
    k[0, 0] = 2.0 ** 24                           # 2**24 + 1 rounds back to 2**24 in binary32
    mu = k_channel_mean(k)
    assert mu[0, 0, 0] == np.float32((2.0 ** 24 + 256) / 512)


def test_k_mean_error_bound_and_constant_channels():
    rng = np.random.default_rng(4)
    for S in (1, 255, 256, 257, 5000):
        k = _bf16(rng.standard_normal((2, S, 3, 128)) * 2 + rng.standard_normal((1, 1, 3, 128)) * 8).float().numpy()
        mu = k_channel_mean(k).astype(np.float64)
        k64 = k.astype(np.float64)
        exact = k64.mean(axis=1)
        nch = -(-S // 256)
        bound = (256 + nch + 2) * U32 * np.abs(k64).sum(axis=1) / S + U32 * np.abs(exact)
        assert np.all(np.abs(mu - exact) <= bound)
    kc = np.full((1, 300, 1, 128), 1.5, np.float32)
    assert np.all(k_channel_mean(kc) == np.float32(1.5))


def test_k_smoothing_leaves_softmax_unchanged():
    q, k, v = _gauss_inputs(1, 70, 2, 2, 5)
    mu = k_channel_mean(k)
    kh = k.float().numpy().astype(np.float64) - mu[:, None, :, :]
    a = exact_attention(q, k, v, 1 / math.sqrt(128))
    b = exact_attention(q, kh, v, 1 / math.sqrt(128))
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- quantizer

@pytest.mark.parametrize("dt,qb,kb", [("int8", 1, 16), ("int8", 4, 4), ("fp8", 1, 4), ("fp8", 16, 1)])
def test_quantizer_roundtrip_bounds(dt, qb, kb):
    q, k, v = _gauss_inputs(1, 203, 4, 2, 6)
    out = sage_quantize(q, k, v, dt, qb, kb)
    qmax = INT8_MAX if dt == "int8" else E4M3_MAX
    khat = (k.float().numpy() - out["mu"][:, None]).astype(np.float32)
    for x, codes, scale, blk in ((q.float().numpy(), out["q_codes"], out["q_scale"], qb),
                                 (khat, out["k_codes"], out["k_scale"], kb)):
        x = x.transpose(0, 2, 1, 3).astype(np.float64)          # [B,H,S,D]
        S = x.shape[2]
        s = np.repeat(scale.astype(np.float64), blk, axis=2)[:, :, :S, None]
        c = _dec(codes, dt)
        err = np.abs(x - c * s)
        if dt == "int8":
            assert np.all(np.abs(c) <= 127)
            # rounding x / s to binary32 first adds at most 2**-24 |x|
            assert np.all(err <= s / 2 + 2.0 ** -23 * np.abs(x))
        else:
            small = np.abs(x) / s < 2.0 ** -6
            assert np.all(err[~small] <= (2.0 ** -4 + 2.0 ** -23) * np.abs(x[~small]))
            assert np.all(err[small] <= 2.0 ** -10 * np.broadcast_to(s, x.shape)[small] + 2.0 ** -23 * np.abs(x[small]))
        # the absmax element of every block maps to +-QMAX
        nb = scale.shape[2]
        for bidx in range(nb):
            blkc = np.abs(c[:, :, bidx * blk:(bidx + 1) * blk])
            assert np.all(blkc.max(axis=(2, 3)) == qmax)
    vx = v.float().numpy().transpose(0, 2, 1, 3).astype(np.float64)
    vc = e4m3_decode(out["v_codes"])
    sv = out["v_scale"][:, :, None, :].astype(np.float64)
    assert np.all(np.abs(vc).max(axis=2) == E4M3_MAX)
    big = np.abs(vx) / sv >= 2.0 ** -6
    assert np.all(np.abs(vx - vc * sv)[big] <= (2.0 ** -4 + 2.0 ** -23) * np.abs(vx)[big])


def test_quantizer_block_scales_brute_force():
    q, k, v = _gauss_inputs(1, 37, 2, 1, 7)
    out = sage_quantize(q, k, v, "int8", 4, 16)
    qx = q.float().numpy()
    for h in range(2):
        for bidx in range(-(-37 // 4)):
            blk = qx[0, bidx * 4:(bidx + 1) * 4, h, :]
            a = max(abs(float(t)) for t in blk.ravel())
            assert out["q_scale"][0, h, bidx] == np.float32(np.float32(a) / np.float32(127))
    vx = v.float().numpy()
    for d in range(128):
        a = max(abs(float(vx[0, s, 0, d])) for s in range(37))
        assert out["v_scale"][0, 0, d] == np.float32(np.float32(a) / np.float32(448))


def test_quantizer_zero_blocks():
    q = torch.zeros((1, 8, 1, 128), dtype=torch.bfloat16)
    k = torch.zeros((1, 8, 1, 128), dtype=torch.bfloat16)
    v = torch.zeros((1, 8, 1, 128), dtype=torch.bfloat16)
    for dt in ("int8", "fp8"):
        out = sage_quantize(q, k, v, dt, 4, 4)
        assert np.all(out["q_scale"] == 1) and np.all(out["k_scale"] == 1) and np.all(out["v_scale"] == 1)
        assert not out["q_codes"].any() and not out["k_codes"].any() and not out["v_codes"].any()


# ---------------------------------------------------------------- exact-code inputs

def _exact_inputs(dt, S, Hq, Hkv, qb, kb, seed):
    """Inputs that every SAGE quantization step maps onto its own codes exactly."""
    rng = np.random.default_rng(seed)
    vals = np.unique(e4m3_decode(np.arange(0x7F, dtype=np.uint8)))
    vals = np.concatenate([-vals, vals])

    def codes(shape):
        if dt == "int8":
            return rng.integers(-127, 128, shape).astype(np.float64)
        return rng.choice(vals, shape)

    qmax = INT8_MAX if dt == "int8" else E4M3_MAX

    def blocked(S, H, blk):
        x = np.zeros((1, S, H, 128))
        for h in range(H):
            for b0 in range(0, S, blk):
                n = min(blk, S - b0)
                c = codes((n, 128))
                c[2 * rng.integers((n + 1) // 2), rng.integers(128)] = qmax * rng.choice([-1, 1])
                x[0, b0:b0 + n, h] = c * 2.0 ** int(rng.integers(-6, 2))
        return x

    q = blocked(S, Hq, qb)
    k = blocked(S, Hkv, kb)
    assert kb in (1, 2, 4, 16) and S % 2 == 0
    # K tokens come in (x, -x) pairs, so every binary32 channel sum stays exactly 0;
    # the forced +-QMAX element sits on an even token, so even-sized blocks keep it
    k[0, 1::2] = -k[0, 0::2]
    v = np.zeros((1, S, Hkv, 128))
    for g in range(Hkv):
        vc = rng.choice(vals, (S, 128))
        vc[rng.integers(S, size=128), np.arange(128)] = E4M3_MAX
        v[0, :, g] = vc * 2.0 ** rng.integers(-5, 3, 128)[None, :]
    for x in (q, k, v):
        assert np.array_equal(_bf16(x).double().numpy(), x)
    return _bf16(q), _bf16(k), _bf16(v)


@pytest.mark.parametrize("dt,qb,kb,Hq,Hkv", [("int8", 1, 16, 2, 2), ("int8", 4, 2, 4, 2),
                                             ("fp8", 1, 4, 3, 1), ("fp8", 16, 16, 2, 1)])
def test_sage_attention_equals_exact_attention_on_exact_codes(dt, qb, kb, Hq, Hkv):
    S = 160
    q, k, v = _exact_inputs(dt, S, Hq, Hkv, qb, kb, 8)
    quant = sage_quantize(q, k, v, dt, qb, kb)
    assert np.all(quant["mu"] == 0)
    sc = 1 / math.sqrt(128)
    got = sage_attention(quant, sc, block_n=64, quantize_p=False)
    ref = exact_attention(q, k, v, sc)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_sage_attention_zero_q_closed_form():
    # Q = 0: every logit is 0, so p = 1 and 2^8 p = 256 is an E4M3 value (no rounding):
    # O = sv_d * mean_j dec(vc_jd) exactly
    _, k, v = _gauss_inputs(1, 150, 2, 1, 9)
    q = torch.zeros((1, 150, 2, 128), dtype=torch.bfloat16)
    quant = sage_quantize(q, k, v, "fp8", 1, 4)
    o = sage_attention(quant, 0.088, block_n=64)
    ref = quant["v_scale"][0, 0].astype(np.float64) * e4m3_decode(quant["v_codes"][0, 0]).mean(axis=0)
    for h in range(2):
        np.testing.assert_allclose(o[0, :, h], np.broadcast_to(ref, (150, 128)), rtol=1e-15, atol=0)


@pytest.mark.parametrize("dt,kb", [("int8", 16), ("fp8", 4)])
def test_sage_attention_constant_v(dt, kb):
    """A V whose rows are all equal (dequantized row u): O = u * (sum_j p~_j / 2^8) /
    (sum_j p_j), and E4M3 rounding of 2^8 p moves each term by at most 2^-4 relative (normal
    range) or 2^-10 absolute (subnormals, p < 2^-14), so |O / u - 1| <= 2^-4 + S 2^-18 / l
    with l >= 1 (the row maximum contributes p = 1).  Without P rounding u comes back up to
    float64 rounding."""
    q, k, _ = _gauss_inputs(1, 200, 2, 1, 12)
    row = torch.randn(128, generator=torch.Generator().manual_seed(3))
    v = row.to(torch.bfloat16)[None, None, None, :].expand(1, 200, 1, 128).contiguous()
    quant = sage_quantize(q, k, v, dt, 1, kb)
    vrow = quant["v_scale"][0, 0].astype(np.float64) * e4m3_decode(quant["v_codes"][0, 0][0])
    o = sage_attention(quant, 1 / math.sqrt(128), block_n=64)
    ratio = o[0] / vrow[None, None, :]
    assert np.all(np.abs(ratio - 1) <= 2.0 ** -4 + 200 * 2.0 ** -18)
    assert np.abs(ratio - 1).max() > 1e-6          # the P rounding is visible
    o2 = sage_attention(quant, 1 / math.sqrt(128), block_n=64, quantize_p=False)
    for h in range(2):
        np.testing.assert_allclose(o2[0, :, h], np.broadcast_to(vrow, (200, 128)), rtol=1e-13, atol=1e-15)


def test_sage_attention_independent_of_tile_size_without_p_rounding():
    q, k, v = _gauss_inputs(1, 200, 2, 2, 10)
    quant = sage_quantize(q, k, v, "int8", 1, 16)
    sc = 1 / math.sqrt(128)
    ref = sage_attention(quant, sc, block_n=200, quantize_p=False)
    for bn in (1, 7, 64, 128):
        np.testing.assert_allclose(sage_attention(quant, sc, block_n=bn, quantize_p=False), ref,
                                   rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("dt,kb", [("int8", 16), ("fp8", 4)])
def test_sage_attention_close_to_exact_attention(dt, kb):
    q, k, v = _gauss_inputs(1, 300, 2, 2, 11)
    quant = sage_quantize(q, k, v, dt, 1, kb)
    sc = 1 / math.sqrt(128)
    ref = exact_attention(q, k, v, sc)
    rel = np.linalg.norm(sage_attention(quant, sc, block_n=64) - ref) / np.linalg.norm(ref)
    rel_nop = np.linalg.norm(sage_attention(quant, sc, block_n=64, quantize_p=False) - ref) / np.linalg.norm(ref)
    # Q/K quantization alone gives 0.028 (int8) / 0.045 (E4M3) on these inputs; the E4M3 P
    # (relative error up to 2^-4 per term, about 2.2e-2 rel-L2 by itself) adds in quadrature
    assert rel_nop < rel < 0.05, (rel_nop, rel)


# ---------------------------------------------------------------- per-element codes, brute force

def _f32(x):
    """Round a Python float to binary32 (nearest-even) through struct."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _ocp_e4m3_table():
    """(value, code) of every finite non-negative OCP E4M3 code, from the format's
    definition: exponent field e (bias 7), mantissa m; e = 0 is subnormal m * 2^-9;
    e = 15, m = 7 is NaN."""
    out = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            val = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
            out.append((val, 8 * e + m))
    return out


E4M3_TABLE = _ocp_e4m3_table()


def _brute_code(x, scale, dt):
    """Code of x in a block with scale `scale`: y = binary32(x / scale) (Python's double
    quotient of two binary32 values, rounded once to binary32: correctly rounded), then
    int8: Python's round (half to even), clamped to +-127; E4M3: the nearest table value,
    ties to the even code, saturated at 448, sign kept (-0 -> 0x80)."""
    y = _f32(x / scale)
    if dt == "int8":
        return max(-127, min(127, round(y)))
    a = min(abs(y), 448.0)
    best = min(E4M3_TABLE, key=lambda vc: (abs(vc[0] - a), vc[1] & 1))
    return best[1] | (0x80 if math.copysign(1.0, y) < 0 else 0)


def _just_below(target, scale):
    """A binary32 x whose exact quotient x / scale lies less than half a binary32 ulp below
    the midpoint `target`: below it in exact (and float64) arithmetic, on it after rounding
    to binary32.  None if no binary32 x near target * scale does that."""
    from fractions import Fraction
    half_ulp = Fraction(float(np.spacing(np.float32(target)))) / 2
    x0 = np.float32(target * scale)
    for cand in (np.nextafter(x0, np.float32(0)), x0, np.nextafter(x0, np.float32(np.inf))):
        qf = Fraction(float(cand)) / Fraction(float(scale))
        if Fraction(target) - half_ulp < qf < Fraction(target):
            return cand
    return None


@pytest.mark.parametrize("dt,qmax,mid,want", [("int8", 127.0, 3.5, 4), ("fp8", 448.0, 1.1875, 0x3A)])
def test_block_codes_brute_force_at_binary32_midpoints(dt, qmax, mid, want):
    """Elements whose exact quotient x / scale sits just below a rounding midpoint (int8:
    3.5; E4M3: 1.1875, between 1.125 (odd mantissa) and 1.25 (even)) but rounds onto it in
    binary32, so round-half-even takes the upper code; a float64 quotient would take the
    lower one.  Every other element of the blocks is checked against the scalar brute force
    too, including -0 and an all-zero block."""
    from oracle.attention import _block_quant_head
    rng = np.random.default_rng(21)
    rows, found = [], 0
    for a in rng.uniform(0.5, 40.0, 400).astype(np.float32):
        scale = np.float32(a / np.float32(qmax))
        x = _just_below(mid, scale)
        if x is None:
            continue
        row = rng.standard_normal(128).astype(np.float32) * np.float32(a / 3)
        row = np.clip(row, -a, a)
        row[0], row[1], row[2], row[3] = a, x, -x, np.float32(-0.0)
        rows.append(row)
        found += 1
        if found == 6:
            break
    assert found == 6
    rows.append(np.zeros(128, np.float32))
    rows[-1][5] = np.float32(-0.0)
    xs = np.stack(rows)
    codes, scales = _block_quant_head(xs, 1, dt)
    for r in range(xs.shape[0]):
        a = float(np.abs(xs[r]).max())
        sc = 1.0 if a == 0 else _f32(a / qmax)
        assert scales[r] == np.float32(sc)
        for d in range(128):
            got = int(codes[r, d]) if dt == "int8" else int(codes[r, d]) & 0xFF
            exp = _brute_code(float(xs[r, d]), sc, dt)
            exp = exp if dt == "int8" else exp & 0xFF
            assert got == exp, (r, d, float(xs[r, d]), got, exp)
    for r in range(found):   # the crafted elements: the upper code, not the float64 one
        if dt == "int8":
            assert codes[r, 1] == want and codes[r, 2] == -want
        else:
            assert codes[r, 1] == want and codes[r, 2] == want | 0x80
        assert (int(codes[r, 3]) & 0xFF) == (0 if dt == "int8" else 0x80)
    assert (int(codes[-1, 5]) & 0xFF) == (0 if dt == "int8" else 0x80)


@pytest.mark.parametrize("dt,blk", [("int8", 4), ("fp8", 16), ("int8", 1), ("fp8", 1)])
def test_block_codes_brute_force_random(dt, blk):
    """Every code and scale of random blocks (including a ragged last block) against the
    scalar brute force."""
    from oracle.attention import _block_quant_head
    rng = np.random.default_rng(22 + blk)
    xs = (rng.standard_normal((37, 128)) * np.exp(rng.uniform(-8, 8, (37, 1)))).astype(np.float32)
    codes, scales = _block_quant_head(xs, blk, dt)
    qmax = 127.0 if dt == "int8" else 448.0
    for b0 in range(0, 37, blk):
        blkx = xs[b0:b0 + blk]
        a = float(np.abs(blkx).max())
        sc = _f32(a / qmax)
        assert scales[b0 // blk] == np.float32(sc)
        for r in range(blkx.shape[0]):
            for d in range(0, 128, 3):
                got = int(codes[b0 + r, d]) if dt == "int8" else int(codes[b0 + r, d]) & 0xFF
                exp = _brute_code(float(blkx[r, d]), sc, dt)
                assert got == (exp if dt == "int8" else exp & 0xFF)

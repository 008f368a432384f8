"""Pins of the oracle's SAGE + Skip-Softmax emulation: reduction to SAGE at
factor 0, equality with the (independently pinned) Skip-Softmax oracle on the
dequantized inputs when P is not rounded, monotone skip sets, and a
constructed case where every later tile is skipped."""
import math

import numpy as np
import pytest

from oracle import e4m3_decode, sage_attention, sage_quantize, sage_skip_attention, skip_attention
from diffusion_transformer_attention_non_amd.synth import positional_qkv

SC = 1 / math.sqrt(128)
BM, BN = 32, 64


@pytest.fixture(scope="module", params=[("int8", 1, 16), ("fp8", 1, 4)])
def peaked_quant(request):
    dt, qb, kb = request.param
    q, k, v = positional_qkv(grid=(2, 8, 24), H=2, seed=5)
    return sage_quantize(q, k, v, dt, qb, kb)


def _dequantized(quant):
    """Q^, K^ (smoothed), V^ in float64, [B, S, H, D], from codes and scales."""
    dt = quant["qk_dtype"]
    dec = (lambda c: c.astype(np.float64)) if dt == "int8" else e4m3_decode
    S = quant["q_codes"].shape[2]
    qs = quant["q_scale"][..., np.arange(S) // quant["q_block"]].astype(np.float64)
    ks = quant["k_scale"][..., np.arange(quant["k_codes"].shape[2]) // quant["k_block"]].astype(np.float64)
    qh = dec(quant["q_codes"]) * qs[..., None]
    kh = dec(quant["k_codes"]) * ks[..., None]
    vh = e4m3_decode(quant["v_codes"]) * quant["v_scale"].astype(np.float64)[:, :, None, :]
    return qh.transpose(0, 2, 1, 3), kh.transpose(0, 2, 1, 3), vh.transpose(0, 2, 1, 3)


def test_factor_zero_is_sage_attention(peaked_quant):
    o, skipped, ratio, rows = sage_skip_attention(peaked_quant, SC, 0.0, BM, BN)
    assert not skipped.any()
    assert np.array_equal(o, sage_attention(peaked_quant, SC, BN, rows=rows))


@pytest.mark.parametrize("factor", [1.0, 10.0, 100.0])
def test_equals_skip_oracle_on_dequantized_inputs_without_p_rounding(peaked_quant, factor):
    """With P unrounded the SAGE emulation is exact softmax attention on the
    dequantized tensors, so skip sets, ratios and outputs must equal those of
    skip_attention on Q^, K^, V^ (K-smoothing shifts each row's logits by a
    constant, which the skip test and softmax ignore)."""
    qh, kh, vh = _dequantized(peaked_quant)
    o, skipped, ratio, rows = sage_skip_attention(peaked_quant, SC, factor, BM, BN, quantize_p=False, p_scale=1.0)
    o_ref, sk_ref, ratio_ref, rows_ref = skip_attention(qh, kh, vh, SC, factor, BM, BN)
    assert np.array_equal(rows, rows_ref)
    lam = factor / qh.shape[1]
    with np.errstate(invalid="ignore"):
        tie = np.abs(np.log2(ratio_ref) - math.log2(lam)) < 1e-9
    assert not tie.any()                      # no decision sits on the threshold
    assert np.array_equal(skipped, sk_ref)
    assert skipped.any()
    np.testing.assert_allclose(ratio, ratio_ref, rtol=1e-9, equal_nan=True)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)


def test_skip_sets_monotone_and_first_tile_kept(peaked_quant):
    prev = None
    for f in (0.5, 1.0, 10.0, 100.0):
        _, sk, _, _ = sage_skip_attention(peaked_quant, SC, f, BM, BN)
        assert not sk[..., 0].any()
        if prev is not None:
            assert np.all(sk >= prev)
        prev = sk
    assert prev.mean() > 0.2


def test_selected_query_tiles_match_full_run(peaked_quant):
    o_all, sk_all, _, _ = sage_skip_attention(peaked_quant, SC, 10.0, BM, BN)
    sel = np.array([1, 4, 11])
    o, sk, _, rows = sage_skip_attention(peaked_quant, SC, 10.0, BM, BN, qtiles=sel)
    assert np.array_equal(sk, sk_all[:, :, sel])
    assert np.array_equal(o, o_all[:, rows])


def test_every_later_tile_skipped_when_maxima_fall():
    """Tile t's logits sit 3t below tile 0's (natural units, sm_scale 1), and
    exp(-3) < lambda = 4 / 64: only tile 0 is kept, so the result is SAGE
    attention over tile 0's keys alone."""
    import torch
    S, bn = 64, 16
    q = torch.zeros(1, S, 1, 128)
    k = torch.zeros(1, S, 1, 128)
    q[0, :, 0, 0] = 1.0
    k[0, :, 0, 0] = torch.from_numpy(-3.0 * (np.arange(S) // bn))
    v = torch.from_numpy(np.random.default_rng(0).standard_normal((1, S, 1, 128)))
    quant = sage_quantize(q.bfloat16(), k.bfloat16(), v.bfloat16(), "int8", 1, 1)
    o, sk, _, rows = sage_skip_attention(quant, 1.0, 4.0, 16, bn)
    assert sk[..., 1:].all() and not sk[..., 0].any()
    first = dict(quant)
    first["k_codes"] = quant["k_codes"][:, :, :bn]
    first["v_codes"] = quant["v_codes"][:, :, :bn]
    first["k_scale"] = quant["k_scale"][:, :, :bn]
    assert np.array_equal(o, sage_attention(first, 1.0, bn))


@pytest.mark.parametrize("delta,skipped", [(-0.01, True), (0.01, False)])
def test_threshold_boundary_in_log2_units(delta, skipped):
    """QK16PV8 codes (exact BF16 values): tile 1's largest logit, in log2 units, sits
    log2(lambda) + delta under tile 0's, lambda = factor / S_kv = 4 / 64; the tile is dropped
    exactly when 2^(M - m) < lambda.  Comparing log2-unit logits with ln(lambda), or a
    threshold without the division by S_kv, puts both cases on the same side."""
    import torch
    S, bn = 64, 32
    lam = 4.0 / S
    q = torch.zeros(1, S, 1, 128)
    k = torch.zeros(1, S, 1, 128)
    v = torch.randn(1, S, 1, 128, generator=torch.Generator().manual_seed(2))
    q[0, :, 0, 0] = 1.0
    k[0, bn:, 0, 0] = -1.0
    sm = -(math.log2(lam) + delta) * math.log(2.0)   # L = sm * (-1) * log2(e) = log2(lam) + delta
    quant = sage_quantize(q.bfloat16(), k.bfloat16(), v.bfloat16(), "bf16", 0, 0, 0)
    _, sk, _, _ = sage_skip_attention(quant, sm, 4.0, 64, bn)
    assert not sk[..., 0].any()
    assert bool(sk[0, 0, 0, 1]) == skipped

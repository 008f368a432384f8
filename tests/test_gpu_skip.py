"""Skip-Softmax attention on the GPU against the oracle's skip emulation."""
import math

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_non_amd as dit
from diffusion_transformer_attention_non_amd.synth import gaussian_qkv, generate, positional_qkv
from oracle import skip_attention
from tests._gpu_util import (announce, compare_skip_sets, dense_tolerances, needs_gpu, parallel_map, ramp_qkv,
                             rel_l2, sample_tiles, to_np)

pytestmark = [pytest.mark.gpu, needs_gpu]
SC = 1 / math.sqrt(128)


def _log_band(q, k):
    """fp32 rounding bound on (M - m) * sm_scale: two logits, each a 128-term
    binary32 dot of exact bf16 products, |error| <= 128 * 2**-24 * sum|q_d k_d|
    <= 128 * 2**-24 * |q| |k| (Cauchy-Schwarz), plus slack for the scaling."""
    qn = float(torch.linalg.vector_norm(q.float(), dim=-1).max())
    kn = float(torch.linalg.vector_norm(k.float(), dim=-1).max())
    return 2 * 128 * 2.0 ** -24 * SC * qn * kn + 4e-7


def _compare_skip_sets(got, ref_skip, ratio, lam, log_band, label=""):
    return compare_skip_sets(got, ref_skip, ratio, lam, log_band, label)


def test_factor_zero_is_bit_identical_to_dense():
    announce("skip factor 0 vs dense")
    q, k, v = positional_qkv(grid=(2, 8, 24), H=2, seed=1)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    dense = dit.attn_dense_bf16(qd, kd, vd)
    o, ex = dit.attn_skip_softmax(qd, kd, vd, 0.0, return_bitmap=True, return_count=True)
    torch.cuda.synchronize()
    assert torch.equal(o, dense)
    assert int(ex["bitmap"].sum()) == 0 and int(ex["skipped"][0]) == 0


@pytest.mark.parametrize("factor", [1.0, 100.0])
def test_bitmap_and_count_do_not_change_the_output(factor):
    """Asking for the bitmap selects another kernel instantiation (the common
    case has no store in its loop): outputs, and LSE, must not depend on it."""
    announce(f"skip output with and without bitmap, factor={factor}")
    q, k, v = positional_qkv(grid=(3, 9, 17), H=3, seed=4)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    plain, ex0 = dit.attn_skip_softmax(qd, kd, vd, factor, return_lse=True)
    counted, ex1 = dit.attn_skip_softmax(qd, kd, vd, factor, return_count=True, return_lse=True)
    mapped, ex2 = dit.attn_skip_softmax(qd, kd, vd, factor, return_bitmap=True, return_count=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(plain, counted) and torch.equal(plain, mapped)
    assert torch.equal(ex0["lse"], ex1["lse"]) and torch.equal(ex0["lse"], ex2["lse"])
    assert int(ex1["skipped"][0]) == int(ex2["skipped"][0]) == int(ex2["bitmap"].sum())
    if factor >= 100.0:
        assert int(ex2["skipped"][0]) > 0


@pytest.mark.parametrize("grid,H,factor", [((2, 8, 24), 2, 1.0), ((2, 8, 24), 2, 10.0), ((2, 8, 24), 2, 100.0),
                                           ((3, 9, 17), 3, 30.0), ((1, 1, 200), 2, 50.0),
                                           # factor above S_kv: lambda = 1000 / 576 > 1, so a half is kept
                                           # only where its maximum rises past the running maximum
                                           ((3, 8, 24), 2, 1000.0)])
def test_skip_set_and_output_match_oracle(grid, H, factor):
    announce(f"skip grid={grid} H={H} factor={factor}")
    bm, bn = dit.tile_config()
    q, k, v = positional_qkv(grid=grid, H=H, seed=2)
    S = q.shape[1]
    o, ex = dit.attn_skip_softmax(q.cuda(), k.cuda(), v.cuda(), factor, out_dtype=torch.float32,
                                  return_bitmap=True, return_count=True)
    torch.cuda.synchronize()
    ref, skipped, ratio, rows = skip_attention(q, k, v, SC, factor, bm, bn)
    got = ex["bitmap"].cpu().numpy().astype(bool)
    assert got.shape == skipped.shape
    band, flips = _compare_skip_sets(got, skipped, ratio, factor / S, _log_band(q, k))
    assert int(ex["skipped"][0]) == int(got.sum())
    assert not got[..., 0].any()
    r = rel_l2(to_np(o)[:, rows], ref)
    assert r <= 3e-2, r
    if flips == 0:
        assert r <= 5e-3, r


def test_gaussian_inputs_rarely_skip_and_stay_exact():
    announce("skip gaussian inputs")
    q, k, v = gaussian_qkv(1, 1000, 2, 1, seed=9)
    o, ex = dit.attn_skip_softmax(q.cuda(), k.cuda(), v.cuda(), 1.0, return_bitmap=True)
    torch.cuda.synchronize()
    bm, bn = dit.tile_config()
    ref, skipped, ratio, rows = skip_attention(q, k, v, SC, 1.0, bm, bn)
    _compare_skip_sets(ex["bitmap"].cpu().numpy().astype(bool), skipped, ratio, 1.0 / 1000, _log_band(q, k))
    assert rel_l2(to_np(o), ref) <= 5e-3


def test_invalid_threshold_rejected():
    q, k, v = gaussian_qkv(1, 8, 1, 1, seed=0)
    for bad in (-1.0, float("nan"), float("inf")):
        with pytest.raises(ValueError, match="THRESHOLD"):
            dit.attn_skip_softmax(q.cuda(), k.cuda(), v.cuda(), bad)


def test_wan_shape_sampled_tiles():
    """B=1, H=40, S=75,600 (21 x 45 x 80 grid), spatially peaked Q/K, factors {0, 1, 10, 100}:
    factor 0 is the dense kernel bit for bit; for the others the skip sets of 8 sampled query
    tiles (first and partial last included) of 4 heads match the oracle outside the tie band
    and the outputs stay within rel-L2 3e-2 of the oracle's restricted softmax."""
    announce("skip wan S=75600 H=40 generate")
    qd, kd, vd = generate("skip_wan_b1_h40_s75600", device="cuda")
    q, k, v = qd.cpu(), kd.cpu(), vd.cpu()
    bm, bn = dit.tile_config()
    S = q.shape[1]
    nqt = -(-S // bm)
    heads = [0, 13, 26, 39]
    qtiles = sample_tiles(nqt, 8, seed=5)
    band = _log_band(q, k)
    announce("skip wan dense")
    dense = dit.attn_dense_bf16(qd, kd, vd)
    for factor in (0.0, 1.0, 10.0, 100.0):
        announce(f"skip wan factor={factor}")
        o, ex = dit.attn_skip_softmax(qd, kd, vd, factor, return_bitmap=True, return_count=True)
        torch.cuda.synchronize()
        bitmap = ex["bitmap"].cpu().numpy().astype(bool)
        assert int(ex["skipped"][0]) == int(bitmap.sum())
        if factor == 0.0:
            assert torch.equal(o, dense) and not bitmap.any()
            continue

        def check(h):
            ref, skipped, ratio, rows = skip_attention(q[:, :, h:h + 1], k[:, :, h:h + 1], v[:, :, h:h + 1], SC,
                                                       factor, bm, bn, qtiles=qtiles)
            _compare_skip_sets(bitmap[:, h:h + 1, qtiles], skipped, ratio, factor / S, band,
                               f"factor={factor} head={h}")
            return rel_l2(to_np(o[:, rows, h:h + 1]), ref)

        for h, r in zip(heads, parallel_map(check, heads)):
            assert r <= 3e-2, (factor, h, r)
        print(f"factor {factor}: skipped fraction {bitmap.mean():.4f}")


def test_gate_routes_dense_before_and_skip_from_the_timestep():
    """The host-side gate of "TRTLLM Attention" (key disabled_until_timestep): with D = 0.86 a
    step at t = 0.9 runs the dense kernel (bit for bit) and steps at t = 0.86 and 0.5 run
    Skip-Softmax (bit for bit the skip call), for BF16 and for SAGE."""
    announce("gate routing")
    q, k, v = positional_qkv(grid=(2, 8, 24), H=2, seed=6)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    gate = dit.SkipGate(0.86)
    dense = dit.attn_dense_bf16(qd, kd, vd)
    skip, ex = dit.attn_skip_softmax(qd, kd, vd, 10.0, return_count=True)
    rec = dit.SageRecipe("fp8", "fp8", 1, 4, 1)
    sage = dit.attn_sage(qd, kd, vd, rec)
    sage_skip, ex2 = dit.attn_sage_skip_softmax(qd, kd, vd, rec, 10.0, return_count=True)
    early = dit.attention(qd, kd, vd, skip_threshold=10.0, gate=gate, timestep=0.9)
    at = dit.attention(qd, kd, vd, skip_threshold=10.0, gate=gate, timestep=0.86)
    late = dit.attention(qd, kd, vd, skip_threshold=10.0, gate=gate, timestep=0.5)
    q_early = dit.attention(qd, kd, vd, quant=rec, skip_threshold=10.0, gate=gate, timestep=0.9)
    q_late = dit.attention(qd, kd, vd, quant=rec, skip_threshold=10.0, gate=gate, timestep=0.5)
    torch.cuda.synchronize()
    assert int(ex["skipped"][0]) > 0 and int(ex2["skipped"][0]) > 0
    assert not torch.equal(dense, skip) and not torch.equal(sage, sage_skip)
    assert torch.equal(early, dense)
    assert torch.equal(at, skip) and torch.equal(late, skip)
    assert torch.equal(q_early, sage) and torch.equal(q_late, sage_skip)


def test_lse_over_kept_keys():
    announce("skip lse")
    q, k, v = positional_qkv(grid=(2, 8, 24), H=2, seed=4)
    bm, bn = dit.tile_config()
    o, ex = dit.attn_skip_softmax(q.cuda(), k.cuda(), v.cuda(), 30.0, out_dtype=torch.float32,
                                  return_bitmap=True, return_lse=True)
    torch.cuda.synchronize()
    ref, skipped, ratio, rows, ref_lse = skip_attention(q, k, v, SC, 30.0, bm, bn, return_lse=True)
    flips = _compare_skip_sets(ex["bitmap"].cpu().numpy().astype(bool), skipped, ratio, 30.0 / q.shape[1],
                               _log_band(q, k))[1]
    if flips == 0:
        err = np.abs(to_np(ex["lse"]) - ref_lse).max()
        assert err <= 4e-3, err


@pytest.mark.parametrize("delta,skipped", [(-0.01, True), (0.01, False)])
def test_threshold_boundary(delta, skipped):
    """The second 32-key half's logits sit ln(lambda) + delta under the first half's (0),
    lambda = factor / S_kv = 4 / 64: the kernel drops the half exactly when exp(M - m) < lambda
    (BF16 inputs are exact here; sm_scale carries the offset)."""
    S = 64
    announce(f"skip threshold boundary delta={delta}")
    q = torch.zeros(1, S, 1, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, S, 1, 128, dtype=torch.bfloat16)
    q[0, :, 0, 0] = 1.0
    k[0, 32:, 0, 0] = -1.0
    v = torch.randn(1, S, 1, 128, generator=torch.Generator().manual_seed(3)).bfloat16()
    sm = -(math.log(4.0 / S) + delta)
    o, ex = dit.attn_skip_softmax(q.cuda(), k.cuda(), v.cuda(), 4.0, sm_scale=sm, return_bitmap=True, return_count=True)
    torch.cuda.synchronize()
    bm = ex["bitmap"].cpu().numpy()
    assert bm.shape[-1] == 2 and bm[0, 0, 0, 0] == 0
    assert bool(bm[0, 0, 0, 1]) == skipped
    assert int(ex["skipped"][0]) == int(skipped)


@pytest.mark.parametrize("sign,factor", [(1.0, 4.0), (-1.0, 4.0), (-1.0, 0.5)])
def test_moving_reference(sign, factor):
    """Logits rising by 0.2 per key over 1,000 keys (no half can be dropped, the lazy
    reference passes its slack on every half) or falling (each half's maximum sits about 6.4
    under the previous one: at lambda = 4 / 1000, exp(-6.4) < lambda and every later half is
    dropped; at lambda = 0.5 / 1000 (ln = -7.6) the second half is kept and the rest, 12.8
    and more under the running maximum, are dropped)."""
    announce(f"skip ramp sign={sign} factor={factor}")
    q, k, v = ramp_qkv(1000, 0.2, seed=13, sign=sign)
    bm, bn = dit.tile_config()
    o, ex = dit.attn_skip_softmax(q.cuda(), k.cuda(), v.cuda(), factor, out_dtype=torch.float32,
                                  return_bitmap=True, return_count=True)
    torch.cuda.synchronize()
    ref, skipped, ratio, rows = skip_attention(q, k, v, SC, factor, bm, bn)
    got = ex["bitmap"].cpu().numpy().astype(bool)
    flips = _compare_skip_sets(got, skipped, ratio, factor / q.shape[1], _log_band(q, k))[1]
    assert int(ex["skipped"][0]) == int(got.sum())
    if sign > 0:
        assert not got.any()
    elif factor == 4.0:
        assert got[..., 1:].all()
    else:
        assert not got[..., 1].any() and got[..., 2:].all()
    if flips == 0:
        dense_tolerances(to_np(o), ref)

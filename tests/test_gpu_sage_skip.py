"""SAGE attention with the Skip-Softmax tile test on the GPU against the
oracle's combined emulation (skip sets compared outside a threshold band)."""
import math

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_non_amd as dit
from diffusion_transformer_attention_non_amd.synth import gaussian_qkv, generate, positional_qkv
from oracle import sage_quantize, sage_skip_attention
from tests._gpu_util import (announce, compare_skip_sets, needs_gpu, parallel_map, ramp_qkv, rel_l2,
                             sample_tiles, to_np)

pytestmark = [pytest.mark.gpu, needs_gpu]
SC = 1 / math.sqrt(128)
LOG2_BAND = 1e-4            # binary32 rounding of L (a scaled int32 or fp32-accumulated dot) in log2 units


def _compare(got, ref_skip, ratio, lam, label=""):
    return compare_skip_sets(got, ref_skip, ratio, lam, LOG2_BAND * math.log(2.0), label)[1]


def _gqa(q, k, v, Hkv):
    """Keep Hkv of the K/V heads (query head h reads KV head h // (Hq / Hkv))."""
    sel = list(range(0, k.shape[2], k.shape[2] // Hkv))[:Hkv]
    return q, k[:, :, sel].contiguous(), v[:, :, sel].contiguous()


@pytest.mark.parametrize("dt,qb,kb", [("int8", 1, 16), ("fp8", 1, 4)])
def test_factor_zero_is_bit_identical_to_sage(dt, qb, kb):
    announce(f"sage-skip factor 0 vs sage {dt}")
    q, k, v = positional_qkv(grid=(2, 8, 24), H=2, seed=1)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    rec = dit.SageRecipe(dt, "fp8", qb, kb, 1)
    ref = dit.attn_sage(qd, kd, vd, rec)
    o, ex = dit.attn_sage_skip_softmax(qd, kd, vd, rec, 0.0, return_bitmap=True, return_count=True)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)
    assert int(ex["bitmap"].sum()) == 0 and int(ex["skipped"][0]) == 0


CASES = [((2, 8, 24), 2, 2, "int8", 1, 16, 1.0), ((2, 8, 24), 2, 2, "fp8", 1, 4, 10.0),
         ((2, 8, 24), 2, 2, "fp8", 1, 1, 100.0), ((3, 9, 17), 4, 2, "int8", 4, 1, 30.0),
         ((1, 1, 200), 2, 1, "fp8", 16, 16, 50.0),
         ((3, 8, 24), 2, 2, "fp8", 1, 4, 1000.0)]   # lambda = 1000 / 576 > 1


@pytest.mark.parametrize("grid,Hq,Hkv,dt,qb,kb,factor", CASES)
def test_skip_set_and_output_match_oracle(grid, Hq, Hkv, dt, qb, kb, factor):
    announce(f"sage-skip grid={grid} Hq={Hq} Hkv={Hkv} {dt} ({qb},{kb}) factor={factor}")
    q, k, v = _gqa(*positional_qkv(grid=grid, H=Hq, seed=2), Hkv)
    S = q.shape[1]
    rec = dit.SageRecipe(dt, "fp8", qb, kb, 1)
    o, ex = dit.attn_sage_skip_softmax(q.cuda(), k.cuda(), v.cuda(), rec, factor, out_dtype=torch.float32,
                                       return_bitmap=True, return_count=True)
    torch.cuda.synchronize()
    bm, _ = dit.sage_skip_tile()
    quant = sage_quantize(q, k, v, dt, qb, kb)
    ref, skipped, ratio, rows = sage_skip_attention(quant, SC, factor, bm, dit.kv_tile())
    got = ex["bitmap"].cpu().numpy().astype(bool)
    assert got.shape == skipped.shape
    flips = _compare(got, skipped, ratio, factor / S)
    assert int(ex["skipped"][0]) == int(got.sum())
    assert not got[..., 0].any()
    assert skipped.any()
    r = rel_l2(to_np(o)[:, rows], ref)
    assert r <= 3e-2, r
    if flips == 0:
        assert r <= 5e-3, r


def test_gaussian_inputs_rarely_skip():
    announce("sage-skip gaussian inputs")
    q, k, v = gaussian_qkv(1, 1000, 2, 1, seed=9, k_bias_std=4.0, outliers=4)
    rec = dit.SageRecipe("fp8", "fp8", 1, 4, 1)
    o, ex = dit.attn_sage_skip_softmax(q.cuda(), k.cuda(), v.cuda(), rec, 1.0, out_dtype=torch.float32,
                                       return_bitmap=True)
    torch.cuda.synchronize()
    quant = sage_quantize(q, k, v, "fp8", 1, 4)
    ref, skipped, ratio, rows = sage_skip_attention(quant, SC, 1.0, *dit.sage_skip_tile())
    flips = _compare(ex["bitmap"].cpu().numpy().astype(bool), skipped, ratio, 1.0 / 1000)
    r = rel_l2(to_np(o), ref)
    assert r <= 3e-2 and (flips or r <= 5e-3), r


def test_invalid_threshold_rejected():
    q, k, v = gaussian_qkv(1, 8, 1, 1, seed=0)
    rec = dit.SageRecipe("int8", "fp8", 1, 16, 1)
    for bad in (-1.0, float("nan"), float("inf")):
        with pytest.raises(ValueError, match="THRESHOLD"):
            dit.attn_sage_skip_softmax(q.cuda(), k.cuda(), v.cuda(), rec, bad)


def test_wan_shape_sampled_tiles():
    """B=1, H=40, S=75,600 (21 x 45 x 80 grid), spatially peaked Q/K, FP8 (1, 4, 1), factors
    {0, 1, 10, 100}: factor 0 is attn_sage bit for bit; otherwise 8 sampled 32-row query blocks
    (first and partial last included) of 4 heads against the combined emulation."""
    announce("sage-skip wan S=75600 H=40 generate")
    qd, kd, vd = generate("skip_wan_b1_h40_s75600", device="cuda")
    q, k, v = qd.cpu(), kd.cpu(), vd.cpu()
    rec = dit.SageRecipe("fp8", "fp8", 1, 4, 1)
    bm, _ = dit.sage_skip_tile()
    S = q.shape[1]
    nqb = -(-S // bm)
    heads = [0, 13, 26, 39]
    qtiles = sample_tiles(nqb, 8, seed=6)
    quants = dict(zip(heads, parallel_map(
        lambda h: sage_quantize(q[:, :, h:h + 1], k[:, :, h:h + 1], v[:, :, h:h + 1], "fp8", 1, 4), heads)))
    announce("sage-skip wan attn_sage")
    plain = dit.attn_sage(qd, kd, vd, rec)
    for factor in (0.0, 1.0, 10.0, 100.0):
        announce(f"sage-skip wan factor={factor}")
        o, ex = dit.attn_sage_skip_softmax(qd, kd, vd, rec, factor, return_bitmap=True, return_count=True)
        torch.cuda.synchronize()
        bitmap = ex["bitmap"].cpu().numpy().astype(bool)
        assert int(ex["skipped"][0]) == int(bitmap.sum())
        if factor == 0.0:
            assert torch.equal(o, plain) and not bitmap.any()
            continue

        def check(h):
            ref, skipped, ratio, rows = sage_skip_attention(quants[h], SC, factor, bm, dit.kv_tile(), qtiles=qtiles)
            _compare(bitmap[:, h:h + 1, qtiles], skipped, ratio, factor / S, f"factor={factor} head={h}")
            return rel_l2(to_np(o[:, rows, h:h + 1]), ref)

        for h, r in zip(heads, parallel_map(check, heads)):
            assert r <= 3e-2, (factor, h, r)
        print(f"factor {factor}: skipped fraction {bitmap.mean():.4f}")


@pytest.mark.parametrize("delta,skipped", [(-0.01, True), (0.01, False)])
def test_threshold_boundary_qk16pv8(delta, skipped):
    """QK16PV8 codes are the exact BF16 inputs: the second 64-key tile's logits sit
    log2(lambda) + delta (log2 units) under the first tile's, lambda = factor / S_kv = 4 / 128;
    the kernel drops the tile exactly when 2^(M - m) < lambda."""
    S = 128
    announce(f"sage skip threshold boundary delta={delta}")
    q = torch.zeros(1, S, 1, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, S, 1, 128, dtype=torch.bfloat16)
    q[0, :, 0, 0] = 1.0
    k[0, 64:, 0, 0] = -1.0
    v = torch.randn(1, S, 1, 128, generator=torch.Generator().manual_seed(4)).bfloat16()
    sm = -(math.log2(4.0 / S) + delta) * math.log(2.0)
    rec = dit.SageRecipe("bf16", "fp8", 0, 0, 0)
    o, ex = dit.attn_sage_skip_softmax(q.cuda(), k.cuda(), v.cuda(), rec, 4.0, sm_scale=sm, return_bitmap=True,
                                       return_count=True)
    torch.cuda.synchronize()
    bm = ex["bitmap"].cpu().numpy()
    assert bm.shape[-1] == 2 and not bm[0, 0, :, 0].any()
    assert np.all(bm[0, 0, :, 1] == int(skipped))


@pytest.mark.parametrize("rec,step", [(("int8", 1, 16, 1), 0.2), (("bf16", 0, 0, 0), 0.2), (("fp8", 1, 4, 1), 0.05)])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_moving_reference(rec, step, sign):
    """Rising logits (no tile can be dropped; the running maximum moves every tile) and
    falling ones (at factor 4 every tile from the third on drops, each sitting at least 9
    log2 units under the running maximum; at step 0.2 the second drops too) through the
    combined kernel."""
    dt, qb, kb, vb = rec
    announce(f"sage-skip ramp {dt} ({qb},{kb},{vb}) step={step} sign={sign}")
    q, k, v = ramp_qkv(1000, step, seed=14, sign=sign)
    r = dit.SageRecipe(dt, "fp8", qb, kb, vb)
    o, ex = dit.attn_sage_skip_softmax(q.cuda(), k.cuda(), v.cuda(), r, 4.0, out_dtype=torch.float32,
                                       return_bitmap=True, return_count=True)
    torch.cuda.synchronize()
    bm, _ = dit.sage_skip_tile()
    quant = sage_quantize(q, k, v, dt, qb, kb, vb)
    ref, skipped, ratio, rows = sage_skip_attention(quant, SC, 4.0, bm, dit.kv_tile())
    got = ex["bitmap"].cpu().numpy().astype(bool)
    flips = _compare(got, skipped, ratio, 4.0 / q.shape[1])
    assert int(ex["skipped"][0]) == int(got.sum())
    if sign > 0:
        assert not skipped.any() and not got.any()
    else:
        assert skipped[..., 2:].all()
    r_ = rel_l2(to_np(o)[:, rows], ref)
    assert r_ <= 3e-2, r_
    if flips == 0 and dt != "fp8":
        assert r_ <= 5e-3, r_

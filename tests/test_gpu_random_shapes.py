"""Seeded random shapes through every attention path against the oracle.

Query and key lengths drawn from [1, 520] (rarely a multiple of the 64-key
tile or of any workgroup height), batch 1-2, KV heads 1-3 and query heads per
KV head 1-3: dense BF16 (output and LSE), BF16 Skip-Softmax (skip set and
output), and SAGE attention for the SageAttention INT8 and FP8 recipes,
MXFP8 Q/K and QK16PV8, each against the oracle's emulation of the same
recipe.  The draws are fixed by the seed, so every run checks the same cases.
"""
import math

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_non_amd as dit
from diffusion_transformer_attention_non_amd.synth import gaussian_qkv
from oracle import exact_attention, sage_attention, sage_quantize, skip_attention
from tests._gpu_util import announce, compare_skip_sets, dense_tolerances, needs_gpu, rel_l2, to_np
from tests.test_gpu_recipes import e4m3_logit_term
from tests.test_gpu_skip import _log_band

pytestmark = [pytest.mark.gpu, needs_gpu]
SC = 1 / math.sqrt(128)


def _cases(n=6, seed=20261202):
    rs = np.random.RandomState(seed)
    out = []
    for _ in range(n):
        hkv = int(rs.randint(1, 4))
        out.append((int(rs.randint(1, 3)), int(rs.randint(1, 521)), int(rs.randint(1, 521)),
                    hkv * int(rs.randint(1, 4)), hkv, float(rs.choice([1.0, 100.0, 1000.0]))))
    return out


CASES = _cases()


def _inputs(B, Sq, Skv, Hq, Hkv):
    q, _, _ = gaussian_qkv(B, Sq, Hq, Hkv, seed=Sq * 7 + Skv)
    _, k, v = gaussian_qkv(B, Skv, Hq, Hkv, seed=Skv * 11 + Sq, k_bias_std=4.0, outliers=4)
    return q, k, v


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,factor", CASES)
def test_dense_and_skip(B, Sq, Skv, Hq, Hkv, factor):
    announce(f"random dense/skip B={B} Sq={Sq} Skv={Skv} Hq={Hq} Hkv={Hkv} factor={factor}")
    q, k, v = _inputs(B, Sq, Skv, Hq, Hkv)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse = dit.attn_dense_bf16(qd, kd, vd, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = exact_attention(q, k, v, SC, return_lse=True)
    dense_tolerances(to_np(o), ref)
    # |LSE| error: the bf16 rounding of P (relative 2^-9 per term) and fp32 sums
    assert np.abs(to_np(lse) - ref_lse).max() <= 4e-3

    bm, bn = dit.tile_config()
    os_, ex = dit.attn_skip_softmax(qd, kd, vd, factor, out_dtype=torch.float32, return_bitmap=True,
                                    return_count=True)
    torch.cuda.synchronize()
    sref, skipped, ratio, rows = skip_attention(q, k, v, SC, factor, bm, bn)
    got = ex["bitmap"].cpu().numpy().astype(bool)
    assert got.shape == skipped.shape
    _, flips = compare_skip_sets(got, skipped, ratio, factor / Skv, _log_band(q, k), f"factor={factor}")
    assert int(ex["skipped"][0]) == int(got.sum())
    r = rel_l2(to_np(os_)[:, rows], sref)
    assert r <= 3e-2, r
    if flips == 0:
        assert r <= 5e-3, r


@pytest.mark.parametrize("rec", [("int8", 1, 16, 1), ("fp8", 1, 4, 1), ("mxfp8", 0, 0, 1), ("bf16", 0, 0, 0)])
@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,factor", CASES[:4])
def test_sage_recipes(rec, B, Sq, Skv, Hq, Hkv, factor):
    announce(f"random sage {rec} B={B} Sq={Sq} Skv={Skv} Hq={Hq} Hkv={Hkv}")
    q, k, v = _inputs(B, Sq, Skv, Hq, Hkv)
    o = dit.attn_sage(q.cuda(), k.cuda(), v.cuda(), dit.SageRecipe(rec[0], "fp8", *rec[1:]), out_dtype=torch.float32)
    torch.cuda.synchronize()
    quant = sage_quantize(q, k, v, *rec)
    emu = sage_attention(quant, SC, dit.kv_tile())
    r = rel_l2(to_np(o), emu)
    # E4M3 Q/K: the matrix core's dot products are not correctly rounded; the bound grows
    # with the logits' size (MXFP8 does not smooth K, so these K-biased inputs reach large
    # ones), as in the recipe tests' accumulation-error model.  0 for INT8 and BF16 Q/K.
    term = e4m3_logit_term(quant, SC)
    print(f"{rec}: rel-L2 {r:.3e}, bound {5e-3 + term:.3e}")
    assert r <= 5e-3 + term, r
    assert r <= 3e-2, r

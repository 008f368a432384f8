"""QK16PV8 and MXFP8 Q/K recipes on the GPU: quantizer bit-exact against the
oracle, attention against the oracle's tile-ordered emulation."""
import math

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_non_amd as dit
from diffusion_transformer_attention_non_amd.synth import gaussian_qkv, generate, positional_qkv
from oracle import exact_attention, sage_attention, sage_quantize, sage_skip_attention
from tests._gpu_util import announce, compare_skip_sets, needs_gpu, ramp_qkv, rel_l2, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]
SC = 1 / math.sqrt(128)
RECIPES = [("bf16", 0, 0, 0), ("mxfp8", 0, 0, 0), ("mxfp8", 0, 0, 1)]


def _check_quant(gpu, ref, S_q, S_kv, dt):
    vc = gpu["v_codes"].cpu().numpy()
    assert np.array_equal(vc[:, :, :, :S_kv].transpose(0, 1, 3, 2), ref["v_codes"])
    assert not vc[:, :, :, S_kv:].any()
    assert np.array_equal(gpu["v_scale"].cpu().numpy(), ref["v_scale"])
    assert not gpu["k_mean"].cpu().numpy().any()
    if dt == "mxfp8":
        qc, kc = gpu["q_codes"].cpu().numpy(), gpu["k_codes"].cpu().numpy()
        assert np.array_equal(qc[:, :, :S_q], ref["q_codes"]) and np.array_equal(kc[:, :, :S_kv], ref["k_codes"])
        assert not qc[:, :, S_q:].any() and not kc[:, :, S_kv:].any()
        qm = gpu["q_mx"].cpu().numpy().astype(np.int64) - 127
        km = gpu["k_mx"].cpu().numpy().astype(np.int64) - 127
        assert np.array_equal(qm[:, :, :S_q], ref["q_scale"]) and np.array_equal(km[:, :, :S_kv], ref["k_scale"])


@pytest.mark.parametrize("rec", RECIPES)
@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv", [(1, 300, 300, 2, 2), (2, 130, 257, 4, 2), (1, 17, 70, 1, 1)])
def test_quantizer_bit_exact(rec, B, Sq, Skv, Hq, Hkv):
    announce(f"quantize {rec} B={B} Sq={Sq} Skv={Skv} Hq={Hq} Hkv={Hkv}")
    q, _, _ = gaussian_qkv(B, Sq, Hq, Hkv, seed=Sq + 1)
    _, k, v = gaussian_qkv(B, Skv, Hq, Hkv, seed=Skv + 2, k_bias_std=4.0, outliers=4)
    q = q * torch.exp(torch.linspace(-6, 6, 128)).to(torch.bfloat16)     # channel blocks of very different size
    r = dit.SageRecipe(rec[0], "fp8", *rec[1:])
    gpu = dit.sage_quantize(q.cuda(), k.cuda(), v.cuda(), r)
    torch.cuda.synchronize()
    _check_quant(gpu, sage_quantize(q, k, v, *rec), Sq, Skv, rec[0])


@pytest.mark.parametrize("rec", RECIPES)
@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv", [(1, 300, 300, 2, 2), (2, 130, 257, 4, 2), (1, 1, 70, 1, 1)])
def test_attention_matches_emulation(rec, B, Sq, Skv, Hq, Hkv):
    announce(f"attention {rec} B={B} Sq={Sq} Skv={Skv} Hq={Hq} Hkv={Hkv}")
    q, _, _ = gaussian_qkv(B, Sq, Hq, Hkv, seed=Sq)
    _, k, v = gaussian_qkv(B, Skv, Hq, Hkv, seed=Skv + 1, k_bias_std=4.0, outliers=4)
    r = dit.SageRecipe(rec[0], "fp8", *rec[1:])
    o = dit.attn_sage(q.cuda(), k.cuda(), v.cuda(), r, out_dtype=torch.float32)
    torch.cuda.synchronize()
    emu = sage_attention(sage_quantize(q, k, v, *rec), SC, dit.kv_tile())
    rr = rel_l2(to_np(o), emu)
    assert rr <= 5e-3, rr
    # sanity against unquantized attention; MXFP8 does not smooth K, so the
    # K bias of these inputs (std 4, outlier channels x8) costs it accuracy
    bar = 0.1 if rec[0] == "bf16" else 0.3
    assert rel_l2(to_np(o), exact_attention(q, k, v, SC)) <= bar


@pytest.mark.parametrize("rec", [("bf16", 0, 0, 0), ("mxfp8", 0, 0, 1)])
def test_skip_softmax_with_recipe_matches_oracle(rec):
    announce(f"skip {rec}")
    q, k, v = positional_qkv(grid=(2, 8, 24), H=2, seed=2)
    r = dit.SageRecipe(rec[0], "fp8", *rec[1:])
    o, ex = dit.attn_sage_skip_softmax(q.cuda(), k.cuda(), v.cuda(), r, 10.0, out_dtype=torch.float32,
                                       return_bitmap=True, return_count=True)
    torch.cuda.synchronize()
    quant = sage_quantize(q, k, v, *rec)
    ref, skipped, ratio, rows = sage_skip_attention(quant, SC, 10.0, *dit.sage_skip_tile())
    got = ex["bitmap"].cpu().numpy().astype(bool)
    flips = compare_skip_sets(got, skipped, ratio, 10.0 / q.shape[1], 1e-4 * math.log(2.0), str(rec))[1]
    assert skipped.any() and int(ex["skipped"][0]) == int(got.sum())
    r_ = rel_l2(to_np(o)[:, rows], ref)
    assert r_ <= 3e-2 and (flips or r_ <= 5e-3), r_


@pytest.mark.parametrize("rec", [("mxfp8", 0, 0, 1), ("bf16", 0, 0, 0)])
def test_wan_shape_sampled(rec):
    """B=1, H=40, S=75,600 Gaussian inputs with K bias and outlier channels: MXFP8 Q/K with
    per-channel V, and QK16PV8 (BF16 Q/K, tensor-wide V scale); sampled rows of two heads."""
    dt, qb, kb, vb = rec
    announce(f"{dt} ({qb},{kb},{vb}) wan generate")
    qd, kd, vd = generate("sage_fp8_wan_b1_h40_s75600", device="cuda")
    r = dit.SageRecipe(dt, "fp8", qb, kb, vb)
    announce(f"{dt} wan attention")
    o = dit.attn_sage(qd, kd, vd, r)
    torch.cuda.synchronize()
    q, k, v = qd.cpu(), kd.cpu(), vd.cpu()
    rows = np.concatenate([np.arange(0, 32), np.arange(40000, 40032), np.arange(75568, 75600)])
    v_amax = float(v.float().abs().max()) if vb == 0 else None   # tensor-wide V scale spans every head
    for h in (0, 39):
        sl = slice(h, h + 1)
        quant = sage_quantize(q[:, :, sl], k[:, :, sl], v[:, :, sl], dt, qb, kb, vb, v_amax=v_amax)
        emu = sage_attention(quant, SC, dit.kv_tile(), rows=rows)
        rr = rel_l2(to_np(o[:, rows, sl]), emu)
        assert rr <= 3e-2, (h, rr)


@pytest.mark.parametrize("rec,step", [(("fp8", 1, 4, 1), 0.05), (("mxfp8", 0, 0, 1), 0.05),
                                      (("int8", 1, 16, 1), 0.2), (("bf16", 0, 0, 0), 0.2),
                                      (("fp8", 1, 4, 1), 0.2), (("mxfp8", 0, 0, 1), 0.2)])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_moving_reference(rec, step, sign):
    """Logits rising over 1,000 keys by `step` per key (natural units; 72 log2 units in all at
    step 0.05, 288 at 0.2): the running maximum moves on every tile and O and the row sums
    are rescaled each time; or falling, so P underflows through the E4M3 subnormals.  The
    bar (rel-L2 3e-2 against the emulation) and the accumulation-error model below are
    asserted wherever the model leaves room for the bar; at step 0.2 the E4M3 Q/K recipes'
    logits reach |L| ~ 400 log2 units, where the E4M3 MFMA's accumulation error alone moves
    the softmax weights by more than the bar allows, so only the model is asserted there."""
    dt, qb, kb, vb = rec
    announce(f"{dt} ({qb},{kb},{vb}) ramp step={step} sign={sign}")
    q, k, v = ramp_qkv(1000, step, seed=12, sign=sign)
    r = dit.SageRecipe(dt, "fp8", qb, kb, vb)
    o = dit.attn_sage(q.cuda(), k.cuda(), v.cuda(), r, out_dtype=torch.float32)
    torch.cuda.synchronize()
    quant = sage_quantize(q, k, v, dt, qb, kb, vb)
    emu = sage_attention(quant, SC, dit.kv_tile())
    rr = rel_l2(to_np(o), emu)
    term = e4m3_logit_term(quant, SC)
    print(f"{rec} step {step} sign {sign}: rel-L2 {rr:.3e}, model bound {5e-3 + term:.3e}")
    assert rr <= 5e-3 + term, rr                            # the accumulation-error model
    if term <= 2.5e-2:
        assert rr <= 3e-2, rr                               # the output bar against the emulation


# The E4M3 MFMA (v_mfma_*_32x32x64_f8f6f4) does not return the correctly rounded sum of its
# 64 exact products: a probe on the device measured errors up to 1.4e-4 of the sum of
# |products| (the BF16 MFMA stays within about 1e-7, the int8 one is exact).  The emulation
# takes exact dot products, so on the E4M3 Q/K paths a logit L_ij (log2 units) may differ
# by up to EPS_E4M3 * sum_d |L-terms|; that moves each softmax weight by a factor within
# 2^(+-2 e_i), e_i the row's largest such bound.
EPS_E4M3 = 2.0 ** -12


def e4m3_logit_term(quant, sm_scale):
    """rms over rows of 2^(2 e_i) - 1 for the E4M3 Q/K formats, 0 for int8 and BF16 Q/K."""
    if quant["qk_dtype"] not in ("fp8", "mxfp8"):
        return 0.0
    from oracle.attention import _logits
    absq = dict(quant, q_codes=quant["q_codes"] & 0x7F, k_codes=quant["k_codes"] & 0x7F)
    B, Hq, Sq, _ = quant["q_codes"].shape
    G = Hq // quant["k_codes"].shape[1]
    rows, keys = np.arange(Sq), np.arange(quant["k_codes"].shape[2])
    terms = []
    for b in range(B):
        for h in range(Hq):
            e = EPS_E4M3 * _logits(absq, b, h, h // G, rows, keys, sm_scale).max(axis=1)
            terms.append(2.0 ** (2 * e) - 1)
    return float(np.sqrt(np.mean(np.concatenate(terms) ** 2)))

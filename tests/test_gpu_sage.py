"""SAGE quantization and attention on the GPU against the oracle."""
import math

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_non_amd as dit
from diffusion_transformer_attention_non_amd.synth import gaussian_qkv, generate
from oracle import exact_attention, sage_attention, sage_quantize
from tests._gpu_util import announce, needs_gpu, rel_l2, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]
SC = 1 / math.sqrt(128)
RECIPES = [("int8", 1, 1), ("int8", 1, 4), ("int8", 1, 16), ("fp8", 1, 1), ("fp8", 1, 4),
           ("int8", 4, 16), ("fp8", 16, 4), ("fp8", 4, 16), ("int8", 16, 1)]


def _check_quant(gpu, ref, S_q, S_kv):
    codes_view = lambda t: t.cpu().numpy()
    qc = codes_view(gpu["q_codes"])
    kc = codes_view(gpu["k_codes"])
    vc = codes_view(gpu["v_codes"])
    assert np.array_equal(qc[:, :, :S_q], ref["q_codes"])
    assert np.array_equal(kc[:, :, :S_kv], ref["k_codes"])
    assert np.array_equal(vc[:, :, :, :S_kv].transpose(0, 1, 3, 2), ref["v_codes"])
    assert not qc[:, :, S_q:].any() and not kc[:, :, S_kv:].any() and not vc[:, :, :, S_kv:].any()
    for name in ("q_scale", "k_scale", "v_scale"):
        assert np.array_equal(gpu[name].cpu().numpy(), ref[name]), name
    assert np.array_equal(gpu["k_mean"].cpu().numpy(), ref["mu"])


@pytest.mark.parametrize("dt,qb,kb", RECIPES)
@pytest.mark.parametrize("S,Hq,Hkv", [(300, 2, 2), (1000, 6, 2), (17, 1, 1)])
def test_quantizer_bit_exact(dt, qb, kb, S, Hq, Hkv):
    announce(f"sage_quantize {dt} ({qb},{kb}) S={S} Hq={Hq} Hkv={Hkv}")
    q, k, v = gaussian_qkv(1, S, Hq, Hkv, seed=S + qb, k_bias_std=4.0, outliers=4)
    rec = dit.SageRecipe(dt, "fp8", qb, kb, 1)
    gpu = dit.sage_quantize(q.cuda(), k.cuda(), v.cuda(), rec)
    torch.cuda.synchronize()
    _check_quant(gpu, sage_quantize(q, k, v, dt, qb, kb), S, S)


@pytest.mark.parametrize("dt,qb,kb", [("int8", 1, 16), ("fp8", 1, 4), ("int8", 4, 1), ("fp8", 16, 16)])
@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv", [(1, 300, 300, 2, 2), (2, 130, 257, 4, 2), (1, 1, 70, 1, 1)])
def test_sage_attention_matches_emulation(dt, qb, kb, B, Sq, Skv, Hq, Hkv):
    announce(f"attn_sage {dt} ({qb},{kb}) B={B} Sq={Sq} Skv={Skv} Hq={Hq} Hkv={Hkv}")
    q, _, _ = gaussian_qkv(B, Sq, Hq, Hkv, seed=Sq)
    _, k, v = gaussian_qkv(B, Skv, Hq, Hkv, seed=Skv + 1, k_bias_std=4.0, outliers=4)
    bn = dit.kv_tile()
    rec = dit.SageRecipe(dt, "fp8", qb, kb, 1)
    o = dit.attn_sage(q.cuda(), k.cuda(), v.cuda(), rec, out_dtype=torch.float32)
    torch.cuda.synchronize()
    quant = sage_quantize(q, k, v, dt, qb, kb)
    emu = sage_attention(quant, SC, bn)
    r = rel_l2(to_np(o), emu)
    assert r <= 3e-2, r
    assert r <= 5e-3, r           # much tighter than the bar in practice
    exact = exact_attention(q, k, v, SC)
    assert rel_l2(to_np(o), exact) <= 0.1


@pytest.mark.parametrize("name", ["sage_int8_b1_h40_s32768", "sage_fp8_wan_b1_h40_s75600"])
def test_full_size_sampled(name):
    from diffusion_transformer_attention_non_amd.synth import WORKLOADS
    w = WORKLOADS[name]
    dt, _, (qb, kb, _) = w.recipe
    announce(f"{name} generate")
    qd, kd, vd = generate(name, device="cuda")
    q, k, v = qd.cpu(), kd.cpu(), vd.cpu()
    rec = dit.SageRecipe(dt, "fp8", qb, kb, 1)
    announce(f"{name} sage_quantize")
    gpu = dit.sage_quantize(qd, kd, vd, rec)
    torch.cuda.synchronize()
    S = q.shape[1]
    bm, _ = dit.tile_config()
    bn = dit.kv_tile()
    nqt = -(-S // bm)
    qtiles = [0, nqt // 3, nqt - 1]
    rows = np.concatenate([np.arange(t * bm, min(S, t * bm + bm)) for t in qtiles])
    announce(f"{name} attn_sage")
    o = dit.attn_sage(qd, kd, vd, rec)
    torch.cuda.synchronize()
    for h in (0, 13, 39):
        sl = slice(h, h + 1)
        ref = sage_quantize(q[:, :, sl], k[:, :, sl], v[:, :, sl], dt, qb, kb)
        sub = {key: (val[:, sl] if isinstance(val, torch.Tensor) and key != "workspace" else val)
               for key, val in gpu.items()}
        _check_quant(sub, ref, S, S)
        emu = sage_attention(ref, SC, bn, rows=rows)
        r = rel_l2(to_np(o[:, rows, sl]), emu)
        assert r <= 3e-2, (h, r)
        print(f"{name} head {h}: rel-L2 vs emulation {r:.2e}")


def test_workspace_too_small_and_bad_recipe():
    q, k, v = gaussian_qkv(1, 64, 1, 1, seed=0)
    rec = dit.SageRecipe("int8", "fp8", 1, 16, 1)
    with pytest.raises(ValueError, match="WORKSPACE"):
        dit.attn_sage(q.cuda(), k.cuda(), v.cuda(), rec, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        dit.SageRecipe("int4", "fp8", 1, 16, 1)

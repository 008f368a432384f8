"""SAGE quantization and attention on the GPU against the oracle."""
import math

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_non_amd as dit
from diffusion_transformer_attention_non_amd.synth import gaussian_qkv, generate
from oracle import exact_attention, sage_attention, sage_quantize
from tests._gpu_util import announce, needs_gpu, parallel_map, rel_l2, sample_tiles, to_np

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
    assert r <= 3e-2, r           # the bar against the oracle's emulation
    assert r <= 5e-3, r           # and a tight one: the kernel takes the emulation's rounding steps
    exact = exact_attention(q, k, v, SC)
    assert rel_l2(to_np(o), exact) <= 0.1


FULL = ["sage_int8_b1_h40_s32768", "sage_fp8_wan_b1_h40_s75600"]


def _full(name):
    from diffusion_transformer_attention_non_amd.synth import WORKLOADS
    dt, _, (qb, kb, _) = WORKLOADS[name].recipe
    announce(f"{name} generate")
    qd, kd, vd = generate(name, device="cuda")
    return qd, kd, vd, dt, qb, kb, dit.SageRecipe(dt, "fp8", qb, kb, 1)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FULL)
def test_full_size_codes_and_scales_all_heads(name):
    """Every code and scale of all 40 heads (Q, K - mean, V, K mean) bit-exact against the
    oracle's quantizer, head by head (every step is per head)."""
    qd, kd, vd, dt, qb, kb, rec = _full(name)
    q, k, v = qd.cpu(), kd.cpu(), vd.cpu()
    announce(f"{name} sage_quantize")
    gpu = dit.sage_quantize(qd, kd, vd, rec)
    torch.cuda.synchronize()
    gpu_np = {key: val.cpu().numpy() for key, val in gpu.items() if isinstance(val, torch.Tensor) and key != "workspace"}
    S = q.shape[1]

    def check(h):
        sl = slice(h, h + 1)
        ref = sage_quantize(q[:, :, sl], k[:, :, sl], v[:, :, sl], dt, qb, kb)
        sub = {key: torch.from_numpy(val[:, sl]) for key, val in gpu_np.items()}
        _check_quant(sub, ref, S, S)
        return h

    assert parallel_map(check, range(q.shape[2])) == list(range(q.shape[2]))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,n_tiles", [(FULL[0], 16), (FULL[1], 8)])
def test_full_size_attention_sampled(name, n_tiles):
    """attn_sage at the full size against the oracle's emulation on sampled 64-row query
    tiles (first and partial last included) of 4 heads, each over the full KV range."""
    qd, kd, vd, dt, qb, kb, rec = _full(name)
    announce(f"{name} attn_sage")
    o = dit.attn_sage(qd, kd, vd, rec)
    torch.cuda.synchronize()
    q, k, v = qd.cpu(), kd.cpu(), vd.cpu()
    S = q.shape[1]
    bm = 64
    qtiles = sample_tiles(-(-S // bm), n_tiles, seed=3)
    rows = np.concatenate([np.arange(t * bm, min(S, t * bm + bm)) for t in qtiles])
    heads = [0, 13, 26, 39]

    def check(h):
        sl = slice(h, h + 1)
        ref = sage_quantize(q[:, :, sl], k[:, :, sl], v[:, :, sl], dt, qb, kb)
        emu = sage_attention(ref, SC, dit.kv_tile(), rows=rows)
        return rel_l2(to_np(o[:, rows, sl]), emu)

    for h, r in zip(heads, parallel_map(check, heads)):
        print(f"{name} head {h}: rel-L2 vs emulation {r:.2e}")
        assert r <= 3e-2, (h, r)
        assert r <= 5e-3, (h, r)


@pytest.mark.parametrize("rec", [("int8", 1, 16, 1), ("fp8", 1, 4, 1), ("fp8", 16, 16, 1), ("int8", 4, 1, 1),
                                 ("mxfp8", 0, 0, 1), ("bf16", 0, 0, 0)])
def test_quantizer_zero_blocks_channels_and_negative_zero(rec):
    """All-zero token blocks of Q, an all-zero K head (mean 0, every block zero), all-zero and
    all-negative-zero V channels, and scattered -0 inputs: scales 1 (MXFP8: exponent -127),
    codes 0 or 0x80 as the sign says, everything else bit-exact; the attention output
    against the emulation as usual."""
    dt, qb, kb, vb = rec
    announce(f"zero blocks {rec}")
    q, k, v = gaussian_qkv(1, 300, 2, 2, seed=40, k_bias_std=2.0)
    q, k, v = q.clone(), k.clone(), v.clone()
    q[:, 32:64] = 0.0                       # whole token blocks of every block size
    q[:, 100:110, 1, :] = -0.0
    k[:, :, 1] = 0.0                        # one K head entirely zero
    k[:, ::7, 1, 5] = -0.0
    v[:, :, 0, 3] = 0.0                     # zero V channel
    v[:, :, 1, 7] = -0.0                    # negative-zero V channel
    v[:, 50:60, 0, 9] = -0.0
    r = dit.SageRecipe(dt, "fp8", qb, kb, vb)
    gpu = dit.sage_quantize(q.cuda(), k.cuda(), v.cuda(), r)
    o = dit.attn_sage(q.cuda(), k.cuda(), v.cuda(), r, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = sage_quantize(q, k, v, dt, qb, kb, vb)
    vc = gpu["v_codes"].cpu().numpy()
    assert np.array_equal(vc[:, :, :, :300].transpose(0, 1, 3, 2), ref["v_codes"])
    assert np.array_equal(gpu["v_scale"].cpu().numpy(), ref["v_scale"])
    assert (ref["v_codes"][0, 1, :, 7] == 0x80).all() and (ref["v_codes"][0, 0, :, 3] == 0).all()
    if dt in ("int8", "fp8"):
        _check_quant(gpu, ref, 300, 300)
        assert (ref["k_scale"][0, 1] == 1).all() and (ref["q_scale"][0, :, 32 // qb:64 // qb] == 1).all()
    elif dt == "mxfp8":
        qm = gpu["q_mx"].cpu().numpy().astype(np.int64) - 127
        km = gpu["k_mx"].cpu().numpy().astype(np.int64) - 127
        assert np.array_equal(qm[:, :, :300], ref["q_scale"]) and np.array_equal(km[:, :, :300], ref["k_scale"])
        assert (ref["k_scale"][0, 1] == -127).all()
        assert np.array_equal(gpu["q_codes"].cpu().numpy()[:, :, :300], ref["q_codes"])
        assert np.array_equal(gpu["k_codes"].cpu().numpy()[:, :, :300], ref["k_codes"])
    emu = sage_attention(ref, SC, dit.kv_tile())
    rr = rel_l2(to_np(o), emu)
    assert rr <= 5e-3, rr


def test_workspace_too_small_and_bad_recipe():
    q, k, v = gaussian_qkv(1, 64, 1, 1, seed=0)
    rec = dit.SageRecipe("int8", "fp8", 1, 16, 1)
    with pytest.raises(ValueError, match="WORKSPACE"):
        dit.attn_sage(q.cuda(), k.cuda(), v.cuda(), rec, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        dit.SageRecipe("int4", "fp8", 1, 16, 1)

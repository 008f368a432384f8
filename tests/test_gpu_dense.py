"""Dense BF16 attention on the GPU against the oracle's exact attention."""
import math

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_non_amd as dit
from diffusion_transformer_attention_non_amd.synth import gaussian_qkv, generate
from oracle import exact_attention
from tests._gpu_util import announce, dense_tolerances, needs_gpu, parallel_map, ramp_qkv, rel_l2, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]
SC = 1 / math.sqrt(128)


def _run(q, k, v, out_dtype=torch.bfloat16):
    return dit.attn_dense_bf16(q.cuda(), k.cuda(), v.cuda(), out_dtype=out_dtype)


def test_small_config_fp32_out_full_parity():
    announce("dense B=1 H=2 S=256 fp32 out")
    q, k, v = generate("dense_b1_h2_s256")
    o = _run(q, k, v, torch.float32)
    torch.cuda.synchronize()
    ref = exact_attention(q, k, v, SC)
    dense_tolerances(to_np(o), ref)


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv", [
    (1, 1, 1, 1, 1), (1, 17, 17, 2, 1), (2, 64, 64, 2, 2), (1, 65, 300, 3, 1),
    (1, 300, 65, 4, 2), (2, 511, 513, 6, 2), (1, 1000, 777, 1, 1), (1, 257, 129, 8, 8)])
def test_ragged_shapes_and_gqa(B, Sq, Skv, Hq, Hkv):
    announce(f"dense B={B} Sq={Sq} Skv={Skv} Hq={Hq} Hkv={Hkv}")
    q, _, _ = gaussian_qkv(B, Sq, Hq, Hkv, seed=Sq + 7 * Skv)
    _, k, v = gaussian_qkv(B, Skv, Hq, Hkv, seed=Skv + 3, k_bias_std=2.0)
    o = _run(q, k, v, torch.float32)
    torch.cuda.synchronize()
    dense_tolerances(to_np(o), exact_attention(q, k, v, SC))


def test_strided_packed_qkv_layout():
    announce("dense packed qkv strides")
    B, S, H = 2, 200, 4
    qkv = torch.randn(B, S, 3, H, 128, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    d = qkv.cuda()
    o = dit.attn_dense_bf16(d[:, :, 0], d[:, :, 1], d[:, :, 2], out_dtype=torch.float32)
    torch.cuda.synchronize()
    dense_tolerances(to_np(o), exact_attention(q, k, v, SC))


def test_bf16_output_is_rounded_fp32_output_and_deterministic():
    announce("dense bf16 vs fp32 output, determinism")
    q, k, v = gaussian_qkv(1, 700, 2, 2, seed=11)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o32 = dit.attn_dense_bf16(qd, kd, vd, out_dtype=torch.float32)
    o16 = dit.attn_dense_bf16(qd, kd, vd)
    o16b = dit.attn_dense_bf16(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(o16, o16b)


def test_gqa_full_size_sampled_rows():
    """B=2, Hq=24, Hkv=8, S=8192 with the per-channel K bias; sampled query rows."""
    announce("dense GQA B=2 Hq=24 Hkv=8 S=8192")
    qd, kd, vd = generate("dense_gqa_b2_h24kv8_s8192", device="cuda")
    q, k, v = qd.cpu(), kd.cpu(), vd.cpu()
    o = dit.attn_dense_bf16(qd, kd, vd)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 8191], np.random.default_rng(0).integers(0, 8192, 40)]))
    ref = exact_attention(q, k, v, SC, rows=rows)
    got = to_np(o)[:, rows]
    dense_tolerances(got, ref)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["skip_wan_b1_h40_s75600", "sage_fp8_wan_b1_h40_s75600"])
def test_wan_shape_sampled_rows(name):
    """B=1, H=40, S=75,600 (the Skip-Softmax workload's spatially peaked inputs, and the
    Gaussian ones with the K bias and outlier channels): sampled rows of the first, a middle
    and the last (partial: 80 rows) 256-row workgroup of 4 heads against exact attention,
    and Skip-Softmax at factor 0 bit-identical to the dense kernel."""
    announce(f"dense wan {name} generate")
    qd, kd, vd = generate(name, device="cuda")
    announce(f"dense wan {name} run")
    o = dit.attn_dense_bf16(qd, kd, vd)
    o0 = dit.attn_skip_softmax(qd, kd, vd, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(o, o0)
    q, k, v = qd.cpu(), kd.cpu(), vd.cpu()
    S = q.shape[1]
    assert S == 75600 and (S - 256 * (S // 256)) == 80
    rows = np.concatenate([np.arange(0, 48), np.arange(37888, 37936), np.arange(75520, 75600)])
    heads = [0, 13, 26, 39]

    def check(h):
        sl = slice(h, h + 1)
        ref = exact_attention(q[:, :, sl], k[:, :, sl], v[:, :, sl], SC, rows=rows)
        return dense_tolerances(to_np(o[:, rows, sl]), ref)

    for h, (ma, rl) in zip(heads, parallel_map(check, heads)):
        print(f"{name} head {h}: max-abs {ma:.2e} rel-L2 {rl:.2e}")


def test_empty_and_invalid_calls():
    announce("dense empty / invalid")
    q, k, v = gaussian_qkv(1, 8, 2, 2, seed=1)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    e = dit.attn_dense_bf16(qd[:, :0], kd, vd)
    assert e.shape == (1, 0, 2, 128)
    with pytest.raises(ValueError, match="S_kv"):
        dit.attn_dense_bf16(qd, kd[:, :0], vd[:, :0])
    with pytest.raises(ValueError, match="HEAD_DIM"):
        dit.attn_dense_bf16(qd[..., :64], kd[..., :64], vd[..., :64])
    with pytest.raises(ValueError, match="GQA"):
        dit.attn_dense_bf16(torch.cat([qd, qd[:, :, :1]], 2), kd, vd)
    with pytest.raises(ValueError):
        dit.attn_dense_bf16(q, k, v)   # host tensors
    with pytest.raises(ValueError, match="mask"):
        dit.attention(qd, kd, vd, attn_mask=torch.ones(8, 8, device="cuda"))


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv", [(1, 300, 65, 4, 2), (2, 130, 513, 2, 2), (1, 1, 1, 1, 1)])
def test_lse_matches_oracle(B, Sq, Skv, Hq, Hkv):
    """Row log-sum-exp next to the output, for self- and cross-attention shapes."""
    announce(f"dense lse B={B} Sq={Sq} Skv={Skv} Hq={Hq} Hkv={Hkv}")
    q, _, _ = gaussian_qkv(B, Sq, Hq, Hkv, seed=Sq + 5)
    _, k, v = gaussian_qkv(B, Skv, Hq, Hkv, seed=Skv + 6, k_bias_std=2.0)
    o, lse = dit.attn_dense_bf16(q.cuda(), k.cuda(), v.cuda(), out_dtype=torch.float32, return_lse=True)
    o_plain = dit.attn_dense_bf16(q.cuda(), k.cuda(), v.cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, ref_lse = exact_attention(q, k, v, SC, return_lse=True)
    dense_tolerances(to_np(o), ref)
    assert torch.equal(o, o_plain)                       # asking for LSE changes nothing else
    # |LSE| error: the bf16 rounding of P (relative 2^-9 per term) and fp32 sums
    err = np.abs(to_np(lse) - ref_lse).max()
    assert err <= 4e-3, err


def test_lse_merges_two_key_halves():
    """LSE-weighted merge of attention over two key halves equals attention over all keys."""
    announce("dense lse merge")
    q, k, v = gaussian_qkv(1, 257, 2, 2, seed=31)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse = dit.attn_dense_bf16(qd, kd, vd, out_dtype=torch.float32, return_lse=True)
    oa, la = dit.attn_dense_bf16(qd, kd[:, :100], vd[:, :100], out_dtype=torch.float32, return_lse=True)
    ob, lb = dit.attn_dense_bf16(qd, kd[:, 100:], vd[:, 100:], out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    wa = torch.exp(la - lse).transpose(1, 2)[..., None]   # [B, Sq, Hq, 1]
    wb = torch.exp(lb - lse).transpose(1, 2)[..., None]
    merged = wa * oa + wb * ob
    assert rel_l2(to_np(merged), to_np(o)) <= 5e-3


@pytest.mark.parametrize("step,sign", [(0.2, 1.0), (0.2, -1.0), (0.02, 1.0)])
def test_moving_reference(step, sign):
    """Row maxima that rise across the whole KV range (the reference moves past the slack
    many times) or fall (every later exponential underflows towards zero)."""
    S = 1000
    announce(f"dense ramp step={step} sign={sign}")
    q, k, v = ramp_qkv(S, step, seed=11, sign=sign)
    o = _run(q, k, v, torch.float32)
    torch.cuda.synchronize()
    dense_tolerances(to_np(o), exact_attention(q, k, v, SC))

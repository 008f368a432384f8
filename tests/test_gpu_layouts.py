"""Layouts and shapes across the entry points on the GPU: packed (strided)
Q/K/V for every recipe, GQA with Skip-Softmax and LSE, and empty problems."""
import math

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_non_amd as dit
from diffusion_transformer_attention_non_amd.synth import gaussian_qkv, positional_qkv
from oracle import exact_attention, sage_attention, sage_quantize, sage_skip_attention, skip_attention
from tests._gpu_util import announce, dense_tolerances, needs_gpu, rel_l2, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]
SC = 1 / math.sqrt(128)


def _packed(B, S, H, seed):
    """Q, K, V as views of one [B, S, 3, H, 128] tensor (row stride 3 H 128)."""
    qkv = torch.randn(B, S, 3, H, 128, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    qkv[:, :, 1] += torch.randn(H, 128, generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16) * 3
    return qkv


@pytest.mark.parametrize("rec", [("int8", 1, 16, 1), ("fp8", 1, 4, 1), ("bf16", 0, 0, 0), ("mxfp8", 0, 0, 1)])
def test_recipes_on_packed_qkv(rec):
    announce(f"packed qkv {rec}")
    B, S, H = 2, 200, 4
    qkv = _packed(B, S, H, 7)
    d = qkv.cuda()
    r = dit.SageRecipe(rec[0], "fp8", *rec[1:])
    o = dit.attn_sage(d[:, :, 0], d[:, :, 1], d[:, :, 2], r, out_dtype=torch.float32)
    torch.cuda.synchronize()
    q, k, v = (qkv[:, :, i].contiguous() for i in range(3))
    emu = sage_attention(sage_quantize(q, k, v, *rec), SC, dit.kv_tile())
    assert rel_l2(to_np(o), emu) <= 5e-3


def test_skip_with_gqa_and_lse():
    announce("skip gqa lse")
    q, k, v = positional_qkv(grid=(2, 8, 24), H=4, seed=11)
    k, v = k[:, :, ::2].contiguous(), v[:, :, ::2].contiguous()        # Hq = 4, Hkv = 2
    bm, bn = dit.tile_config()
    o, ex = dit.attn_skip_softmax(q.cuda(), k.cuda(), v.cuda(), 30.0, out_dtype=torch.float32,
                                  return_bitmap=True, return_count=True, return_lse=True)
    torch.cuda.synchronize()
    ref, skipped, ratio, rows, ref_lse = skip_attention(q, k, v, SC, 30.0, bm, bn, return_lse=True)
    got = ex["bitmap"].cpu().numpy().astype(bool)
    lam = 30.0 / q.shape[1]
    with np.errstate(divide="ignore", invalid="ignore"):
        near = np.abs(np.log(ratio) - math.log(lam)) <= 1e-4
    assert not ((got != skipped) & ~near).any()
    assert skipped.any() and int(ex["skipped"][0]) == int(got.sum())
    if not ((got != skipped) & near).any():
        assert rel_l2(to_np(o)[:, rows], ref) <= 5e-3
        assert np.abs(to_np(ex["lse"]) - ref_lse).max() <= 4e-3


def test_dense_lse_with_gqa_and_strides():
    announce("dense lse gqa strided")
    qkv = _packed(1, 150, 4, 13)
    d = qkv.cuda()
    k, v = d[:, :, 1, ::2], d[:, :, 2, ::2]                               # Hkv = 2, non-contiguous head stride
    o, lse = dit.attn_dense_bf16(d[:, :, 0], k, v, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    q = qkv[:, :, 0].contiguous()
    kc, vc = qkv[:, :, 1, ::2].contiguous(), qkv[:, :, 2, ::2].contiguous()
    ref, ref_lse = exact_attention(q, kc, vc, SC, return_lse=True)
    dense_tolerances(to_np(o), ref)
    assert np.abs(to_np(lse) - ref_lse).max() <= 4e-3


def test_empty_problems_launch_nothing():
    announce("empty problems")
    q, k, v = gaussian_qkv(1, 8, 2, 2, seed=1)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    rec = dit.SageRecipe("fp8", "fp8", 1, 4, 1)
    assert dit.attn_sage(qd[:, :0], kd, vd, rec).shape == (1, 0, 2, 128)
    o, ex = dit.attn_sage_skip_softmax(qd[:, :0], kd, vd, rec, 1.0, return_count=True)
    assert o.shape == (1, 0, 2, 128)
    o, ex = dit.attn_skip_softmax(qd[:, :0], kd, vd, 1.0, return_count=True, return_lse=True)
    assert o.shape == (1, 0, 2, 128) and ex["lse"].shape == (1, 2, 0)
    torch.cuda.synchronize()


def test_hip_graph_capture_and_replay():
    """The entry points enqueue kernels only (no allocation, memset or synchronisation in
    the library), so a captured sequence of dense, SAGE and Skip-Softmax calls replays to
    the eager results, replay after replay, with other work on the device in between."""
    announce("hip graph capture of dense + sage + skip")
    q, k, v = gaussian_qkv(1, 700, 4, 2, seed=21, k_bias_std=2.0)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    rec = dit.SageRecipe("fp8", "fp8", 1, 4, 1)
    ws = dit.sage_workspace(q, k, v, rec)
    outs = [torch.empty(q.shape, dtype=torch.bfloat16, device="cuda") for _ in range(3)]

    def calls():
        dit.attn_dense_bf16(q, k, v, out=outs[0])
        dit.attn_sage(q, k, v, rec, out=outs[1], workspace=ws)
        dit.attn_skip_softmax(q, k, v, 10.0, out=outs[2])

    calls()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for i in range(3):
        for o in outs:
            o.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda") * (i + 1)       # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), i
        del junk


def test_concurrent_streams():
    """Calls on two streams run concurrently and stay independent (the library keeps no
    device state between calls; each SAGE call has its own workspace)."""
    announce("dense + sage on two streams")
    q1, k1, v1 = (t.cuda() for t in gaussian_qkv(1, 900, 4, 2, seed=31))
    q2, k2, v2 = (t.cuda() for t in gaussian_qkv(2, 500, 2, 1, seed=32, k_bias_std=3.0))
    rec = dit.SageRecipe("int8", "fp8", 1, 16, 1)
    ref1 = dit.attn_dense_bf16(q1, k1, v1)
    ref2 = dit.attn_sage(q2, k2, v2, rec)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            o1 = dit.attn_dense_bf16(q1, k1, v1)
        with torch.cuda.stream(s2):
            o2 = dit.attn_sage(q2, k2, v2, rec)
        outs.append((o1, o2))
    torch.cuda.synchronize()
    for o1, o2 in outs:
        assert torch.equal(o1, ref1) and torch.equal(o2, ref2)

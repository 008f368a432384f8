"""The C-ABI library on the CPU: exported symbols, host-only queries, and
argument validation (every check runs before any device call)."""
import ctypes
import os
import re
import subprocess

import pytest

import diffusion_transformer_attention_non_amd as dit
from diffusion_transformer_attention_non_amd import _Layout, _Recipe, _Shape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ditattn.h")
GOLDEN_RECIPES = os.path.join(ROOT, "tests", "golden", "trtllm_sage_recipes.txt")
GOLDEN_CUTEDSL = os.path.join(ROOT, "tests", "golden", "cutedsl_recipes.txt")

OK, INVALID, HEAD_DIM, GQA, RECIPE, LAYOUT, THRESHOLD, WS, DEVICE = 0, -1, -2, -3, -4, -5, -6, -7, -8

lib_missing = not os.path.exists(dit.library_path())
pytestmark = pytest.mark.skipif(lib_missing, reason="libditattn.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert "attn_dense_bf16" in names and "attn_sage_skip_softmax" in names and len(names) == 11
    out = subprocess.run(["nm", "-D", "--defined-only", dit.library_path()], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(dit.library_path())
    for n in names:
        assert hasattr(lib, n)


def test_host_queries():
    assert dit.tile_config() == (64, 32)
    assert dit.sage_skip_tile() == (32, 64)
    assert dit.kv_tile() == 64
    assert dit._lib().attn_version() >= 100


@pytest.mark.parametrize("t,D,on", [(1.0, 1.0, True), (0.86, 0.86, True), (0.9, 0.86, False), (0.0, 0.0, True),
                                    (0.01, 0.0, False), (0.5, 1.0, True)])
def test_skip_gate(t, D, on):
    assert dit.SkipGate(D).enabled(t) is on


@pytest.mark.parametrize("t,D", [(1.5, 0.5), (-0.1, 0.5), (0.5, float("nan")), (float("inf"), 0.5)])
def test_skip_gate_rejects(t, D):
    with pytest.raises(ValueError):
        dit.SkipGate(D).enabled(t)


def _shape(B=1, S=256, Hq=2, Hkv=2, D=128, Skv=None):
    s = _Shape(B=B, S_q=S, S_kv=S if Skv is None else Skv, Hq=Hq, Hkv=Hkv, D=D)
    for f, H in (("q_stride", Hq), ("k_stride", Hkv), ("v_stride", Hkv), ("o_stride", Hq)):
        getattr(s, f)[:] = [S * H * D, H * D, D]
    return s


FAKE = ctypes.c_void_p(0x100000)


def _dense(shape, o_dtype=0, scale=0.088):
    return dit._lib().attn_dense_bf16(FAKE, FAKE, FAKE, FAKE, o_dtype, ctypes.byref(shape), scale, None, None)


def test_dense_validation_codes():
    assert _dense(_shape(D=64)) == HEAD_DIM
    assert _dense(_shape(Hq=3, Hkv=2)) == GQA
    assert _dense(_shape(Hkv=0)) == GQA
    assert _dense(_shape(B=-1)) == INVALID
    assert _dense(_shape(), o_dtype=2) == INVALID
    assert _dense(_shape(), scale=0.0) == INVALID
    assert _dense(_shape(), scale=float("nan")) == INVALID
    s = _shape()
    s.q_stride[1] = 129
    assert _dense(s) == LAYOUT
    assert _dense(_shape(S=0)) == OK               # empty problem: nothing to do
    assert _dense(_shape(Skv=0)) == INVALID        # softmax over no keys
    lib = dit._lib()
    assert lib.attn_dense_bf16(None, FAKE, FAKE, FAKE, 0, ctypes.byref(_shape()), 0.1, None, None) == INVALID
    assert lib.attn_dense_bf16(ctypes.c_void_p(0x100008), FAKE, FAKE, FAKE, 0, ctypes.byref(_shape()), 0.1, None,
                               None) == LAYOUT
    assert b"16-byte" in lib.attn_last_error()
    assert lib.attn_dense_bf16(FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(_shape()), 0.1, ctypes.c_void_p(0x200002),
                               None) == LAYOUT
    assert b"lse" in lib.attn_last_error()


def test_valid_call_without_gpu_reports_device_error():
    rc = _dense(_shape())
    if rc != DEVICE:
        pytest.skip("a GPU is present")
    assert dit._lib().attn_last_error()


def test_skip_threshold_validation():
    lib = dit._lib()
    for bad in (-1.0, float("nan"), float("inf")):
        assert lib.attn_skip_softmax(FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(_shape()), 0.1, bad, None, None, None,
                                     None) == THRESHOLD


def _recipe(qk, qb, kb, v=3, vb=1):
    return _Recipe(qk_dtype=qk, v_dtype=v, q_block=qb, k_block=kb, v_block=vb)


def _layout(shape, rec):
    lay = _Layout()
    rc = dit._lib().attn_sage_layout_query(ctypes.byref(shape), ctypes.byref(rec), ctypes.byref(lay))
    return rc, lay


def test_recipes_listed_on_the_pages_are_accepted():
    names = {"int8": 2, "fp8": 3}
    n = 0
    for line in open(GOLDEN_RECIPES):
        if line.startswith("#") or not line.strip():
            continue
        qk, v, qb, kb, vb = line.split()
        rc, _ = _layout(_shape(), _recipe(names[qk], int(qb), int(kb), names[v], int(vb)))
        assert rc == OK, line
        dit.SageRecipe(qk, v, int(qb), int(kb), int(vb))
        n += 1
    assert n == 5
    for qk in (2, 3):        # the key tables also allow q and k blocks of 1, 4 and 16 each
        for qb in (1, 4, 16):
            for kb in (1, 4, 16):
                assert _layout(_shape(), _recipe(qk, qb, kb))[0] == OK


def test_bf16_and_mxfp8_recipes_listed_on_the_pages_are_accepted():
    names = {"bf16": 0, "mxfp8": 4, "fp8": 3}
    n = 0
    for line in open(GOLDEN_CUTEDSL):
        if line.startswith("#") or not line.strip():
            continue
        qk, v, qb, kb, vb = line.split()
        rc, lay = _layout(_shape(S=300), _recipe(names[qk], int(qb), int(kb), names[v], int(vb)))
        assert rc == OK, line
        dit.SageRecipe(qk, v, int(qb), int(kb), int(vb))
        if qk == "bf16":      # no Q/K codes or scales
            assert lay.n_qblk == 0 and lay.k_codes_off == lay.q_codes_off and lay.v_codes_off == lay.k_codes_off
        else:                 # one 4-byte word of E8M0 scales per token row
            assert lay.n_qblk == lay.s_pad == 320 and lay.n_kblk == 320
        n += 1
    assert n == 3


@pytest.mark.parametrize("qk,qb,kb,v,vb", [(0, 1, 16, 3, 1), (1, 1, 16, 3, 1), (2, 2, 16, 3, 1), (2, 1, 8, 3, 1),
                                           (3, 1, 32, 3, 1), (2, 1, 16, 2, 1), (2, 1, 16, 3, 0), (2, 0, 16, 3, 1),
                                           (0, 0, 0, 3, 1), (4, 0, 0, 3, 2), (4, 1, 0, 3, 0), (4, 0, 0, 4, 0),
                                           (5, 0, 0, 3, 0)])
def test_other_recipes_are_rejected(qk, qb, kb, v, vb):
    assert _layout(_shape(), _recipe(qk, qb, kb, v, vb))[0] == RECIPE


@pytest.mark.parametrize("kw", [dict(qk_dtype="int4"), dict(v_dtype="int8"), dict(q_block=2), dict(k_block=32),
                                dict(v_block=0), dict(q_block=True), dict(qk_dtype="bf16"),
                                dict(qk_dtype="mxfp8", q_block=0, k_block=0, v_block=2)])
def test_python_recipe_validation(kw):
    with pytest.raises(ValueError):
        dit.SageRecipe(**kw)


def test_sage_layout_arithmetic():
    s = _shape(B=2, S=1000, Hq=6, Hkv=2, Skv=700)
    rc, L = _layout(s, _recipe(2, 4, 16))
    assert rc == OK
    assert L.s_pad == 1024 and L.n_qblk == 250 and L.n_kblk == 44
    offs = [L.q_codes_off, L.k_codes_off, L.v_codes_off, L.q_scale_off, L.k_scale_off, L.v_scale_off,
            L.k_mean_off, L.scratch_off]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
    assert L.k_codes_off - L.q_codes_off >= 2 * 6 * 1024 * 128
    assert L.v_codes_off - L.k_codes_off >= 2 * 2 * 1024 * 128
    assert L.q_scale_off - L.v_codes_off >= 2 * 2 * 128 * 1024
    assert L.k_scale_off - L.q_scale_off >= 4 * 2 * 6 * 250
    assert L.total_bytes > L.scratch_off + 4 * 2 * 2 * 3 * 128


def test_sage_workspace_checked_before_device():
    lib = dit._lib()
    s = _shape()
    rec = _recipe(2, 1, 16)
    ws = ctypes.c_void_p(0x200000)
    assert lib.sage_quantize(FAKE, FAKE, FAKE, ctypes.byref(s), ctypes.byref(rec), ws, 10, None) == WS
    assert lib.sage_quantize(FAKE, FAKE, FAKE, ctypes.byref(s), ctypes.byref(rec), None, 1 << 30, None) == INVALID
    assert lib.sage_quantize(FAKE, FAKE, FAKE, ctypes.byref(s), ctypes.byref(rec), ctypes.c_void_p(0x200010), 1 << 30,
                             None) == LAYOUT
    assert lib.attn_sage(FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(s), ctypes.byref(_recipe(2, 3, 16)), 0.1, ws, 1 << 30,
                         None) == RECIPE


def test_sage_skip_threshold_and_workspace_checked_before_device():
    lib = dit._lib()
    s = _shape()
    rec = _recipe(2, 1, 16)
    ws = ctypes.c_void_p(0x200000)
    F = ctypes.c_float
    call = lambda factor, wsb=1 << 30, r=rec: lib.attn_sage_skip_softmax(
        FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(s), ctypes.byref(r), F(0.1), F(factor), None, None, ws, wsb, None)
    assert call(-1.0) == THRESHOLD
    assert call(float("nan")) == THRESHOLD
    assert call(float("inf")) == THRESHOLD
    assert call(1.0, wsb=10) == WS
    assert call(1.0, r=_recipe(2, 3, 16)) == RECIPE


def test_size_limits_rejected_before_device():
    lib = dit._lib()
    big = 1 << 31
    assert _dense(_shape(S=big)) == INVALID
    assert b"too large" in lib.attn_last_error()
    assert _dense(_shape(B=1 << 16, Hq=1 << 15, Hkv=1 << 15)) == INVALID
    assert _dense(_shape(S=1 << 30, Hq=1 << 9, Hkv=1 << 9)) == INVALID   # 2^31 workgroups
    assert b"one launch" in lib.attn_last_error()
    # one head's K rows span (S_kv + 256) * k_stride[1] * 2 bytes through 32-bit offsets
    s = _shape(S=1 << 24, Hq=1, Hkv=1)
    assert _dense(s) == INVALID
    assert b"4 GiB" in lib.attn_last_error()
    s = _shape(S=(1 << 24) - 512, Hq=1, Hkv=1)
    assert _dense(s) in (DEVICE, OK)               # inside the limit: only the device check remains
    # the quantized path: codes of one head through 32-bit offsets
    rec = _recipe(3, 1, 4)
    ws = ctypes.c_void_p(0x100000)
    s = _shape(S=1 << 25, Hq=1, Hkv=1)
    rc = lib.attn_sage(FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(s), ctypes.byref(rec), ctypes.c_float(0.088),
                       ws, ctypes.c_size_t(1 << 62), None)
    assert rc == INVALID
    assert b"4 GiB" in lib.attn_last_error()


def test_overlapping_rows_rejected_before_device():
    s = _shape()
    s.k_stride[1] = 0                     # a broadcast K view: every row reads the same place
    assert _dense(s) == LAYOUT
    s = _shape()
    s.v_stride[1] = 64
    assert _dense(s) == LAYOUT
    s = _shape(S=1)
    s.k_stride[1] = 0                     # even with one key: the kernels size views from it
    assert _dense(s) == LAYOUT
    s = _shape()
    s.o_stride[:] = [256 * 2 * 128, 128, 128]   # o rows of different heads collide
    assert _dense(s) == LAYOUT
    s = _shape()
    s.o_stride[:] = [0, 2 * 128, 128]     # B = 1: the batch stride does not matter
    assert _dense(s) == DEVICE
    s = _shape()
    s.o_stride[:] = [256 * 2 * 128, 128, 256 * 128]   # [B, H, S, D] output: fine
    assert _dense(s) == DEVICE
    s = _shape()
    s.q_stride[1] = 0                     # Q is only read: a broadcast query is allowed
    assert _dense(s) == DEVICE


@pytest.mark.parametrize("bad", [-1.0, float("nan"), float("inf"), "x"])
def test_attention_router_rejects_bad_threshold_before_routing(bad):
    import torch
    q = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)   # host tensors: nothing is launched
    with pytest.raises(ValueError, match="skip_threshold"):
        dit.attention(q, q, q, skip_threshold=bad)


def test_noalloc_quantizer_limits_checked_before_device():
    """The static statistics scratch is 16 MiB: 40 KV heads at S_kv = 300,000 (1,172 chunks of
    256 tokens per head) need about 24 MB and are refused before any device call; the
    output region must hold the layout's scratch_off bytes."""
    lib = dit._lib()
    rec = _Recipe(qk_dtype=3, v_dtype=3, q_block=1, k_block=4, v_block=1)
    big = _shape(S=300000, Hq=40, Hkv=40)
    assert lib.sage_quantize_noalloc(FAKE, FAKE, FAKE, ctypes.byref(big), ctypes.byref(rec), FAKE,
                                     1 << 40, None) == WS
    assert "static scratch" in lib.attn_last_error().decode()
    s = _shape(S=1000)
    lay = _Layout()
    assert lib.attn_sage_layout_query(ctypes.byref(s), ctypes.byref(rec), ctypes.byref(lay)) == OK
    assert lib.sage_quantize_noalloc(FAKE, FAKE, FAKE, ctypes.byref(s), ctypes.byref(rec), FAKE,
                                     lay.scratch_off - 1, None) == WS
    assert lib.sage_quantize_noalloc(FAKE, FAKE, FAKE, ctypes.byref(s), ctypes.byref(rec), FAKE,
                                     lay.scratch_off, None) == DEVICE

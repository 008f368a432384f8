"""sage_quantize_noalloc on the GPU, called through the C ABI: the same codes,
scales and K mean as sage_quantize, bit for bit, on two calls in a row (the
second one smaller, so it runs on the static scratch the first one left)."""
import ctypes

import pytest
import torch

import diffusion_transformer_attention_non_amd as dit
from diffusion_transformer_attention_non_amd import _views
from diffusion_transformer_attention_non_amd.synth import gaussian_qkv
from tests._gpu_util import announce, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]

RECIPES = [("int8", 1, 16, 1), ("fp8", 1, 4, 1), ("fp8", 16, 1, 1), ("mxfp8", 0, 0, 1), ("mxfp8", 0, 0, 0),
           ("bf16", 0, 0, 0)]


def _c_call(name, q, k, v, rec, buf):
    shape = dit._shape(q, k, v)
    rc = getattr(dit._lib(), name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(shape),
                                   ctypes.byref(rec._c()), buf.data_ptr(), buf.numel(),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, (name, rc, dit._lib().attn_last_error())


@pytest.mark.parametrize("rec", RECIPES)
def test_noalloc_matches_sage_quantize_on_two_calls(rec):
    r = dit.SageRecipe(rec[0], "fp8", *rec[1:])
    for B, S, Hq, Hkv, seed in ((2, 3000, 6, 3, 1), (1, 300, 2, 1, 2)):   # the second call is smaller
        announce(f"noalloc {rec} B={B} S={S} Hq={Hq} Hkv={Hkv}")
        q, k, v = gaussian_qkv(B, S, Hq, Hkv, seed=seed, k_bias_std=4.0, outliers=4)
        q, k, v = q.cuda(), k.cuda(), v.cuda()
        lay = dit._layout(q, k, v, r)
        ws = torch.full((lay.total_bytes,), 0x5A, dtype=torch.uint8, device="cuda")
        out = torch.full((lay.scratch_off,), 0xA5, dtype=torch.uint8, device="cuda")
        _c_call("sage_quantize", q, k, v, r, ws)
        _c_call("sage_quantize_noalloc", q, k, v, r, out)
        torch.cuda.synchronize()
        ref, got = _views(ws, lay, q, k, r), _views(out, lay, q, k, r)
        for key, val in ref.items():
            if isinstance(val, torch.Tensor) and key != "workspace":
                assert torch.equal(got[key], val), (rec, S, key)

"""Non-causal fused attention for diffusion transformers on AMD MI355X (gfx950).

Python binding of ``libditattn.so`` (C ABI in ``include/ditattn.h``).  This
layer only marshals arguments: tensors come from PyTorch (device memory and
the current stream); every step of the computation runs in the library's HIP
kernels.  There is no CPU or PyTorch fallback: if the library is missing the
calls raise.

Entry points (same names as the C ABI):
  attn_dense_bf16(q, k, v)                 dense BF16 attention
  sage_quantize(q, k, v, recipe)           SAGE codes and scales
  sage_quantize_noalloc(q, k, v, recipe)   the same, statistics in a static scratch
  attn_sage(q, k, v, recipe)               SAGE attention
  attn_skip_softmax(q, k, v, factor)       Skip-Softmax attention
  attn_sage_skip_softmax(q, k, v, recipe, factor)   SAGE with Skip-Softmax
  SkipGate(D).enabled(t)                   host-side timestep gate
  attention(...)                           one call that routes a DiT layer

Pages followed (titles as published): "TRTLLM Attention" (vllm-omni user
guide), "Diffusion Attention Backends", "SAGE + Skip-Softmax - API Design &
Test Plan", "VisualGen Quantized Attention (Beta)".
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

__all__ = [
    "AttnError", "SageRecipe", "SkipGate", "attn_dense_bf16", "sage_quantize", "sage_quantize_noalloc",
    "attn_sage", "attn_skip_softmax", "attn_sage_skip_softmax", "attention", "tile_config",
    "kv_tile", "sage_skip_tile", "library_path",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libditattn.so")

ATTN_OK = 0
_STATUS = {
    -1: "INVALID_ARG", -2: "UNSUPPORTED_HEAD_DIM", -3: "BAD_GQA", -4: "UNSUPPORTED_RECIPE",
    -5: "BAD_LAYOUT", -6: "BAD_THRESHOLD", -7: "WORKSPACE_TOO_SMALL", -8: "DEVICE",
    -9: "NOT_IMPLEMENTED",
}
_VALIDATION = {-1, -2, -3, -4, -5, -6, -7}
DT_BF16, DT_FP32, DT_INT8, DT_FP8, DT_MXFP8 = 0, 1, 2, 3, 4


class AttnError(RuntimeError):
    """A device-side failure reported by the library."""


class _Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("S_q", ctypes.c_int64), ("S_kv", ctypes.c_int64),
                ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64), ("D", ctypes.c_int64),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
                ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3)]


class _Recipe(ctypes.Structure):
    _fields_ = [("qk_dtype", ctypes.c_int), ("v_dtype", ctypes.c_int), ("q_block", ctypes.c_int32),
                ("k_block", ctypes.c_int32), ("v_block", ctypes.c_int32)]


class _Layout(ctypes.Structure):
    _fields_ = [("total_bytes", ctypes.c_size_t), ("q_codes_off", ctypes.c_size_t),
                ("k_codes_off", ctypes.c_size_t), ("v_codes_off", ctypes.c_size_t),
                ("q_scale_off", ctypes.c_size_t), ("k_scale_off", ctypes.c_size_t),
                ("v_scale_off", ctypes.c_size_t), ("k_mean_off", ctypes.c_size_t),
                ("scratch_off", ctypes.c_size_t), ("s_pad", ctypes.c_int64),
                ("n_qblk", ctypes.c_int64), ("n_kblk", ctypes.c_int64)]


_lib_handle = None


def library_path() -> str:
    return _LIB_PATH


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built: run `python -m diffusion_transformer_attention_non_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        SP, RP, LP = ctypes.POINTER(_Shape), ctypes.POINTER(_Recipe), ctypes.POINTER(_Layout)
        sig = {
            "attn_dense_bf16": [P, P, P, P, I, SP, F, P, P],
            "attn_sage_layout_query": [SP, RP, LP],
            "sage_quantize": [P, P, P, SP, RP, P, ctypes.c_size_t, P],
            "sage_quantize_noalloc": [P, P, P, SP, RP, P, ctypes.c_size_t, P],
            "attn_sage": [P, P, P, P, I, SP, RP, F, P, ctypes.c_size_t, P],
            "attn_skip_softmax": [P, P, P, P, I, SP, F, F, P, P, P, P],
            "attn_sage_skip_softmax": [P, P, P, P, I, SP, RP, F, F, P, P, P, ctypes.c_size_t, P],
            "attn_skip_gate": [F, F, ctypes.POINTER(I)],
            "attn_tile_config": [ctypes.POINTER(I)] * 4,
            "attn_version": [],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = I
        lib.attn_last_error.argtypes = []
        lib.attn_last_error.restype = ctypes.c_char_p
        _lib_handle = lib
    return _lib_handle


def _check(rc: int):
    if rc == ATTN_OK:
        return
    msg = _lib().attn_last_error().decode(errors="replace")
    name = _STATUS.get(rc, str(rc))
    if rc in _VALIDATION:
        raise ValueError(f"ATTN_ERR_{name}: {msg}")
    raise AttnError(f"ATTN_ERR_{name}: {msg}")


def _tiles():
    v = [ctypes.c_int() for _ in range(4)]
    _check(_lib().attn_tile_config(*(ctypes.byref(x) for x in v)))
    return [x.value for x in v]


def tile_config():
    """(block_m, block_n): query rows and keys per BF16 Skip-Softmax vote."""
    bm, bn, _, _ = _tiles()
    return bm, bn


def kv_tile():
    """Keys per KV tile of the online softmax (SAGE's P rounding follows it)."""
    return _tiles()[2]


def sage_skip_tile():
    """(rows, keys) per vote of SAGE + Skip-Softmax: one KV tile of keys."""
    _, _, kv, sbm = _tiles()
    return sbm, kv


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check_tensors(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch.Tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, S, H, D], got {tuple(t.shape)}")
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.stride(-1) != 1 and t.shape[-1] > 1:
            raise ValueError(f"{name} must have a contiguous last (head_dim) axis")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on one device")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if q.shape[0] != k.shape[0] or q.shape[3] != k.shape[3]:
        raise ValueError("q and k must agree on batch and head_dim")


def _shape(q, k, v, o=None) -> _Shape:
    """The C shape; without an output (quantization only) O's strides are those
    of a contiguous [B, S_q, Hq, D] tensor."""
    B, Sq, Hq, D = q.shape
    _, Skv, Hkv, _ = k.shape
    s = _Shape(B=B, S_q=Sq, S_kv=Skv, Hq=Hq, Hkv=Hkv, D=D)
    for field, t in (("q_stride", q), ("k_stride", k), ("v_stride", v)):
        getattr(s, field)[:] = [t.stride(0), t.stride(1), t.stride(2)]
    s.o_stride[:] = [o.stride(0), o.stride(1), o.stride(2)] if o is not None else [Sq * Hq * D, Hq * D, D]
    return s


def _out(q, out, out_dtype):
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if out.shape != q.shape or out.device != q.device or out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out must match q's shape and device and be bfloat16 or float32")
    if out.stride(-1) != 1:
        raise ValueError("out must have a contiguous last axis")
    return out, (DT_FP32 if out.dtype == torch.float32 else DT_BF16)


def _scale(q, sm_scale):
    return 1.0 / math.sqrt(q.shape[-1]) if sm_scale is None else float(sm_scale)


def _lse_buffer(q, want):
    if not want:
        return None
    B, Sq, Hq, _ = q.shape
    return torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)


def attn_dense_bf16(q, k, v, out=None, out_dtype=torch.bfloat16, sm_scale=None, return_lse=False):
    """Dense non-causal attention softmax(sm_scale Q K^T) V, BF16 inputs.

    With ``return_lse`` returns (out, lse), lse [B, Hq, S_q] float32 holding
    ln sum_j exp(sm_scale <q_i, k_j>) per row.
    """
    _check_tensors(q, k, v)
    out, odt = _out(q, out, out_dtype)
    shape = _shape(q, k, v, out)
    lse = _lse_buffer(q, return_lse)
    _check(_lib().attn_dense_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), odt,
                                  ctypes.byref(shape), _scale(q, sm_scale),
                                  lse.data_ptr() if lse is not None else None, _stream(q)))
    return (out, lse) if return_lse else out


@dataclass(frozen=True)
class SageRecipe:
    """(qk_dtype, v_dtype, (q_block, k_block, v_block)), validated like the pages' recipe table.

    SageAttention: qk_dtype "int8" or "fp8" / "fp8_e4m3", q_block, k_block in
    {1, 4, 16} tokens, v_block = 1 (one V scale per head and channel).
    QK16PV8: qk_dtype "bf16", blocks (0, 0, 0) (tensor-wide V scale).
    MXFP8 Q/K: qk_dtype "mxfp8", blocks (0, 0, 0) or (0, 0, 1).
    v_dtype is "fp8" throughout.
    """
    qk_dtype: str = "int8"
    v_dtype: str = "fp8"
    q_block: int = 1
    k_block: int = 16
    v_block: int = 1

    def __post_init__(self):
        if self.v_dtype not in ("fp8", "fp8_e4m3"):
            raise ValueError(f"v_dtype must be 'fp8', got {self.v_dtype!r}")
        blocks = (self.q_block, self.k_block, self.v_block)
        if any(isinstance(x, bool) for x in blocks):
            raise ValueError(f"block sizes must be integers, got {blocks!r}")
        if self.qk_dtype in ("int8", "fp8", "fp8_e4m3"):
            for name in ("q_block", "k_block"):
                if getattr(self, name) not in (1, 4, 16):
                    raise ValueError(f"{name} must be 1, 4 or 16, got {getattr(self, name)!r}")
            if self.v_block != 1:
                raise ValueError("v_block must be 1 (per-channel V scale)")
        elif self.qk_dtype == "bf16":
            if blocks != (0, 0, 0):
                raise ValueError(f"the QK16PV8 recipe takes blocks (0, 0, 0), got {blocks!r}")
        elif self.qk_dtype == "mxfp8":
            if blocks not in ((0, 0, 0), (0, 0, 1)):
                raise ValueError(f"the MXFP8 Q/K recipe takes blocks (0, 0, 0) or (0, 0, 1), got {blocks!r}")
        else:
            raise ValueError(f"qk_dtype must be 'int8', 'fp8_e4m3', 'bf16' or 'mxfp8', got {self.qk_dtype!r}")

    @property
    def int8(self) -> bool:
        return self.qk_dtype == "int8"

    def _c(self) -> _Recipe:
        qk = {"int8": DT_INT8, "bf16": DT_BF16, "mxfp8": DT_MXFP8}.get(self.qk_dtype, DT_FP8)
        return _Recipe(qk_dtype=qk, v_dtype=DT_FP8, q_block=self.q_block, k_block=self.k_block,
                       v_block=self.v_block)


def _layout(q, k, v, recipe: SageRecipe):
    shape = _shape(q, k, v)
    lay = _Layout()
    _check(_lib().attn_sage_layout_query(ctypes.byref(shape), ctypes.byref(recipe._c()), ctypes.byref(lay)))
    return lay


def sage_workspace(q, k, v, recipe: SageRecipe) -> torch.Tensor:
    """A uint8 device buffer large enough for sage_quantize / attn_sage."""
    lay = _layout(q, k, v, recipe)
    return torch.empty(max(1, lay.total_bytes), dtype=torch.uint8, device=q.device)


def sage_quantize(q, k, v, recipe: SageRecipe, workspace=None):
    """Quantize Q, K (smoothed) and V; returns views of the codes and scales.

    Keys of the result: q_codes [B,Hq,s_pad,128], k_codes [B,Hkv,s_pad,128],
    v_codes [B,Hkv,128,s_pad] (d-major), q_scale [B,Hq,n_qblk],
    k_scale [B,Hkv,n_kblk], v_scale [B,Hkv,128], k_mean [B,Hkv,128],
    s_pad, workspace.  Codes are int8 (int8 recipe) or uint8 E4M3 bits.
    """
    _check_tensors(q, k, v)
    lay = _layout(q, k, v, recipe)
    if workspace is None:
        workspace = torch.empty(max(1, lay.total_bytes), dtype=torch.uint8, device=q.device)
    shape = _shape(q, k, v)
    _check(_lib().sage_quantize(q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(shape),
                                ctypes.byref(recipe._c()), workspace.data_ptr(), workspace.numel(), _stream(q)))
    return _views(workspace, lay, q, k, recipe)


def sage_quantize_noalloc(q, k, v, recipe: SageRecipe, out=None):
    """sage_quantize whose statistics scratch lives in the library's static
    device array (the C call allocates nothing).  ``out``: a uint8 device
    buffer of at least the layout's ``scratch_off`` bytes (allocated here if
    not given).  Returns the same views as sage_quantize."""
    _check_tensors(q, k, v)
    lay = _layout(q, k, v, recipe)
    if out is None:
        out = torch.empty(max(1, lay.scratch_off), dtype=torch.uint8, device=q.device)
    shape = _shape(q, k, v)
    _check(_lib().sage_quantize_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(shape),
                                        ctypes.byref(recipe._c()), out.data_ptr(), out.numel(), _stream(q)))
    return _views(out, lay, q, k, recipe)


def _views(ws, lay, q, k, recipe):
    B, Sq, Hq, D = q.shape
    Hkv = k.shape[2]
    sp = lay.s_pad

    def region(off, n, dtype, shape):
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return ws[off:off + nbytes].view(dtype).view(shape)

    cdt = torch.int8 if recipe.int8 else torch.uint8
    views = {
        "v_codes": region(lay.v_codes_off, B * Hkv * D * sp, torch.uint8, (B, Hkv, D, sp)),
        "v_scale": region(lay.v_scale_off, B * Hkv * D, torch.float32, (B, Hkv, D)),
        "k_mean": region(lay.k_mean_off, B * Hkv * D, torch.float32, (B, Hkv, D)),
        "s_pad": sp,
        "workspace": ws,
    }
    if recipe.qk_dtype != "bf16":
        views["q_codes"] = region(lay.q_codes_off, B * Hq * sp * D, cdt, (B, Hq, sp, D))
        views["k_codes"] = region(lay.k_codes_off, B * Hkv * sp * D, cdt, (B, Hkv, sp, D))
    if recipe.qk_dtype == "mxfp8":   # E8M0 bytes, one per 32 channels of a token
        views["q_mx"] = region(lay.q_scale_off, B * Hq * sp * 4, torch.uint8, (B, Hq, sp, 4))
        views["k_mx"] = region(lay.k_scale_off, B * Hkv * sp * 4, torch.uint8, (B, Hkv, sp, 4))
    elif recipe.qk_dtype != "bf16":
        views["q_scale"] = region(lay.q_scale_off, B * Hq * lay.n_qblk, torch.float32, (B, Hq, lay.n_qblk))
        views["k_scale"] = region(lay.k_scale_off, B * Hkv * lay.n_kblk, torch.float32, (B, Hkv, lay.n_kblk))
    return views


def attn_sage(q, k, v, recipe: SageRecipe = SageRecipe(), out=None, out_dtype=torch.bfloat16,
              sm_scale=None, workspace=None):
    """Low-precision attention for a recipe: SageAttention (K-smoothing inside),
    QK16PV8 or MXFP8 Q/K; quantize, then attention with an FP8 BMM2."""
    _check_tensors(q, k, v)
    out, odt = _out(q, out, out_dtype)
    lay = _layout(q, k, v, recipe)
    if workspace is None:
        workspace = torch.empty(max(1, lay.total_bytes), dtype=torch.uint8, device=q.device)
    shape = _shape(q, k, v, out)
    _check(_lib().attn_sage(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), odt, ctypes.byref(shape),
                            ctypes.byref(recipe._c()), _scale(q, sm_scale), workspace.data_ptr(),
                            workspace.numel(), _stream(q)))
    return out


def attn_skip_softmax(q, k, v, threshold_factor, out=None, out_dtype=torch.bfloat16, sm_scale=None,
                      return_bitmap=False, return_count=False, return_lse=False):
    """Skip-Softmax attention with threshold = threshold_factor / S_kv.

    Returns out, or (out, extras) with extras holding "bitmap" (uint8
    [B, Hq, ceil(S_q/block_m), ceil(S_kv/block_n)], 1 = skipped), "skipped"
    (a one-element int64 tensor) and/or "lse" ([B, Hq, S_q] float32, over the
    kept keys) when requested.
    """
    _check_tensors(q, k, v)
    out, odt = _out(q, out, out_dtype)
    shape = _shape(q, k, v, out)
    bm, bn = tile_config()
    bitmap = cnt = None
    if return_bitmap:
        B, Sq, Hq, _ = q.shape
        bitmap = torch.empty((B, Hq, -(-Sq // bm), -(-k.shape[1] // bn)), dtype=torch.uint8, device=q.device)
    if return_count:
        cnt = torch.empty(1, dtype=torch.int64, device=q.device)
    lse = _lse_buffer(q, return_lse)
    _check(_lib().attn_skip_softmax(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), odt,
                                    ctypes.byref(shape), _scale(q, sm_scale), float(threshold_factor),
                                    bitmap.data_ptr() if bitmap is not None else None,
                                    cnt.data_ptr() if cnt is not None else None,
                                    lse.data_ptr() if lse is not None else None, _stream(q)))
    if not (return_bitmap or return_count or return_lse):
        return out
    extras = {}
    if bitmap is not None:
        extras["bitmap"] = bitmap
    if cnt is not None:
        extras["skipped"] = cnt
    if lse is not None:
        extras["lse"] = lse
    return out, extras


def attn_sage_skip_softmax(q, k, v, recipe: SageRecipe, threshold_factor, out=None, out_dtype=torch.bfloat16,
                           sm_scale=None, workspace=None, return_bitmap=False, return_count=False):
    """SAGE attention with the Skip-Softmax tile test (threshold_factor / S_kv)
    on its dequantized logits, in one kernel.

    The vote tile is ``sage_skip_tile()``: 32 query rows x one 64-key KV tile.  Returns out, or (out, extras) as attn_skip_softmax.
    """
    _check_tensors(q, k, v)
    out, odt = _out(q, out, out_dtype)
    lay = _layout(q, k, v, recipe)
    if workspace is None:
        workspace = torch.empty(max(1, lay.total_bytes), dtype=torch.uint8, device=q.device)
    shape = _shape(q, k, v, out)
    bm, kv = sage_skip_tile()
    bitmap = cnt = None
    if return_bitmap:
        B, Sq, Hq, _ = q.shape
        bitmap = torch.empty((B, Hq, -(-Sq // bm), -(-k.shape[1] // kv)), dtype=torch.uint8, device=q.device)
    if return_count:
        cnt = torch.empty(1, dtype=torch.int64, device=q.device)
    _check(_lib().attn_sage_skip_softmax(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), odt,
                                         ctypes.byref(shape), ctypes.byref(recipe._c()), _scale(q, sm_scale),
                                         float(threshold_factor),
                                         bitmap.data_ptr() if bitmap is not None else None,
                                         cnt.data_ptr() if cnt is not None else None,
                                         workspace.data_ptr(), workspace.numel(), _stream(q)))
    if not (return_bitmap or return_count):
        return out
    extras = {}
    if bitmap is not None:
        extras["bitmap"] = bitmap
    if cnt is not None:
        extras["skipped"] = cnt
    return out, extras


class SkipGate:
    """Host-side gate: Skip-Softmax runs on a step iff its normalized timestep t <= D.

    t runs from 1 (noisiest, first step) to 0; D = disabled_until_timestep in
    [0, 1].  The gate has no kernel argument: a step it disables runs dense.
    """

    def __init__(self, disabled_until_timestep: float):
        self.D = float(disabled_until_timestep)
        self.enabled(1.0)   # validates D

    def enabled(self, t: float) -> bool:
        flag = ctypes.c_int()
        _check(_lib().attn_skip_gate(float(t), self.D, ctypes.byref(flag)))
        return bool(flag.value)


def attention(q, k, v, *, quant: SageRecipe | None = None, skip_threshold: float | None = None,
              gate: SkipGate | None = None, timestep: float | None = None, attn_mask=None,
              out=None, out_dtype=torch.bfloat16, sm_scale=None):
    """One DiT attention call: dense, SAGE, Skip-Softmax (when the gate
    allows), or SAGE with Skip-Softmax.

    ``skip_threshold`` is the threshold factor (lambda = factor / S_kv): finite
    and >= 0, 0 meaning no skipping; anything else raises ValueError before
    any routing.  With a ``gate``, a step whose normalized ``timestep`` is
    above the gate's value runs without Skip-Softmax.  A mask is refused: this
    backend only serves mask-free layers.
    """
    if attn_mask is not None:
        raise ValueError("attention masks are not supported: this path is mask-free only")
    if skip_threshold is not None:
        try:
            factor = float(skip_threshold)
        except (TypeError, ValueError):
            raise ValueError(f"skip_threshold must be a real number, got {skip_threshold!r}") from None
        if not (math.isfinite(factor) and factor >= 0.0):
            raise ValueError(f"skip_threshold must be finite and >= 0, got {skip_threshold!r}")
    use_skip = skip_threshold is not None and float(skip_threshold) > 0.0
    if use_skip and gate is not None:
        if timestep is None:
            raise ValueError("a gated Skip-Softmax call needs the normalized timestep")
        use_skip = gate.enabled(timestep)
    if quant is not None and use_skip:
        return attn_sage_skip_softmax(q, k, v, quant, skip_threshold, out=out, out_dtype=out_dtype,
                                      sm_scale=sm_scale)
    if quant is not None:
        return attn_sage(q, k, v, quant, out=out, out_dtype=out_dtype, sm_scale=sm_scale)
    if use_skip:
        return attn_skip_softmax(q, k, v, skip_threshold, out=out, out_dtype=out_dtype, sm_scale=sm_scale)
    return attn_dense_bf16(q, k, v, out=out, out_dtype=out_dtype, sm_scale=sm_scale)

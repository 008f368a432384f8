"""Oracle attention: exact softmax attention, SAGE quantization and its
attention emulation, Skip-Softmax emulation, and the timestep gate.

TEST INFRASTRUCTURE ONLY (see the package header).

Layouts: Q is [B, S_q, Hq, D], K and V are [B, S_kv, Hkv, D], D = 128, with
query head h reading KV head h // (Hq // Hkv) ("GQA native" in the backend
table of "Diffusion Attention Backends"; consecutive grouping is the reading
taken here).  Attention is non-causal and unmasked (TRTLLM Attention,
"Requirements": a packed or mask-free path).

Parity status:
  exact_attention   pinned: brute force on tiny shapes, torch SDPA in float64,
                    closed forms (constant V, Q = 0, one dominant key),
                    permutation invariance, rows of P summing to 1; its LSE
                    against scipy's logsumexp and ln(S_kv) at Q = 0.
  k_channel_mean    pinned: closed-form error bound against the float64 mean,
                    exact on constant channels.
  sage_quantize     pinned: softmax invariance of the smoothing, round-trip
                    error bounds, absmax element -> +-QMAX, zero blocks,
                    per-block brute force on tiny inputs.
  sage_quantize     also pinned: every per-element code against a scalar
                    brute force (Python division rounded to binary32, round
                    half to even, nearest-value search over the OCP E4M3 table).
  sage_attention    pinned: Q = 0 closed form, equality with exact attention
                    on exactly representable inputs with P rounding off,
                    independence of the KV tile size with P rounding off;
                    two-key closed forms (one tile, and one key per tile with
                    the maximum moving); the error bound for a constant V.
  sage_skip_attention pinned: factor 0 equals sage_attention bit for bit;
                    with P rounding off, skip set and output equal
                    skip_attention on the dequantized inputs; monotone in the
                    factor; first tile never skipped; a dominant first tile
                    skips every later one.
  skip_attention    pinned: factor 0 equals exact attention (LSE too), monotone skip
                    sets, first tile never skipped, scalar brute force on tiny
                    grids, dropped-mass error bound, a constructed case where
                    every later tile is skipped.
  skip_gate_enabled pinned: truth table.
The constants that the pages do not fix (QMAX values, rounding mode, the 2**8
P scale, the KV-mean summation order, tile sizes) are readings, checked only
by the invariants above: "parity unpinned by the pages" for those constants.
"""
from __future__ import annotations

import math

import numpy as np

from .codecs import E4M3_MAX, INT8_MAX, e4m3_decode, e4m3_encode, f32, int8_code, bf16_round

MEAN_CHUNK = 256
_ROW_CHUNK_ELEMS = 1 << 25


def _f64(x):
    if hasattr(x, "detach"):            # a torch tensor (bfloat16 is exact in float32)
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def _f32(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float32)


def _shape_check(q, k, v):
    B, Sq, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    if (Bk, Dk) != (B, D) or tuple(v.shape) != tuple(k.shape) or Hq % Hkv:
        raise ValueError("bad attention shapes")
    return B, Sq, Skv, Hq, Hkv, D


def _round_out(o, out_dtype):
    if out_dtype is None:
        return o
    if out_dtype == "bf16":
        return bf16_round(o)
    if out_dtype == "fp32":
        return f32(o).astype(np.float64)
    raise ValueError(out_dtype)


# ----------------------------------------------------------------------------
# Exact attention
# ----------------------------------------------------------------------------

def exact_attention(q, k, v, sm_scale, rows=None, out_dtype=None, return_probs=False, return_lse=False):
    """O = softmax(sm_scale * Q K^T) V per (batch, query head), in float64.

    The plain definition of the fused multi-head attention that the pages'
    dense mode computes ("TRTLLM Attention", section "Dense mode"): for each
    query row i, s_ij = sm_scale * <q_i, k_j>, p_ij = exp(s_ij - max_j s_ij),
    O_i = sum_j p_ij v_j / sum_j p_ij, over every key j (non-causal, no mask).

    ``rows`` selects query rows (the same for every batch entry and head).
    Returns O as [B, R, Hq, D] float64, and with ``return_probs`` also the
    normalized probabilities [B, Hq, R, S_kv]; with ``return_lse`` also the
    row log-sum-exp LSE_i = ln sum_j exp(s_ij) [B, Hq, R] (natural log, the
    quantity that merges partial attention results over key subsets).
    """
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    B, Sq, Skv, Hq, Hkv, D = _shape_check(qf, kf, vf)
    G = Hq // Hkv
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    R = len(rows)
    out = np.empty((B, R, Hq, D))
    probs = np.empty((B, Hq, R, Skv)) if return_probs else None
    lse = np.empty((B, Hq, R))
    step = max(1, _ROW_CHUNK_ELEMS // max(1, Skv))
    for b in range(B):
        for h in range(Hq):
            kg, vg = kf[b, :, h // G, :], vf[b, :, h // G, :]
            for r0 in range(0, R, step):
                rr = rows[r0:r0 + step]
                s = sm_scale * (qf[b, rr, h, :] @ kg.T)
                mx = s.max(axis=1, keepdims=True)
                p = np.exp(s - mx)
                l = p.sum(axis=1, keepdims=True)
                out[b, r0:r0 + step, h, :] = (p @ vg) / l
                lse[b, h, r0:r0 + step] = (mx + np.log(l))[:, 0]
                if return_probs:
                    probs[b, h, r0:r0 + step, :] = p / l
    out = _round_out(out, out_dtype)
    res = (out,) + ((probs,) if return_probs else ()) + ((lse,) if return_lse else ())
    return res if len(res) > 1 else out


# ----------------------------------------------------------------------------
# SAGE quantization
# ----------------------------------------------------------------------------

def k_channel_mean(k):
    """K-smoothing mean mu[b, g, d] over all S_kv tokens, binary32, pinned order.

    The pages say only that K-smoothing is internal ("TRTLLM Attention",
    section "SAGE quantization"; "Diffusion Attention Backends", section
    "TRTLLM_ATTN SAGE Quantization").  Reading: subtract the per-channel mean
    of K over every token of a (batch, KV head), which leaves softmax
    unchanged.  Summation order (pinned so a GPU can match it bit for bit):
    tokens are cut into chunks of 256; inside a chunk a binary32 accumulator
    starting at +0 adds the tokens in ascending order; the chunk sums are then
    added in ascending chunk order into a binary32 total starting at +0; the
    mean is total / binary32(S_kv), correctly rounded.
    """
    kf = _f32(k)
    B, S, H, D = kf.shape
    nch = -(-S // MEAN_CHUNK)
    pad = nch * MEAN_CHUNK - S
    if pad:   # adding +0.0 to an accumulator that started at +0 changes nothing
        kf = np.concatenate([kf, np.zeros((B, pad, H, D), np.float32)], axis=1)
    kc = kf.reshape(B, nch, MEAN_CHUNK, H, D)
    acc = np.zeros((B, nch, H, D), np.float32)
    for j in range(MEAN_CHUNK):
        acc = acc + kc[:, :, j]
    tot = np.zeros((B, H, D), np.float32)
    for c in range(nch):
        tot = tot + acc[:, c]
    return tot / np.float32(S)


def _qmax(dtype):
    if dtype == "int8":
        return np.float32(INT8_MAX)
    if dtype in ("fp8", "fp8_e4m3"):
        return np.float32(E4M3_MAX)
    raise ValueError(f"unsupported qk dtype {dtype!r}")


def _encode(y, dtype):
    return int8_code(y) if dtype == "int8" else e4m3_encode(y)


def _decode(c, dtype):
    if dtype in ("int8", "bf16"):
        return c.astype(np.float64)
    return e4m3_decode(c)


def _block_quant_head(x, blk, dtype):
    """Per-token-block quantization of one [S, D] binary32 slice.

    A block is ``blk`` consecutive tokens x all D channels (the last block
    takes what is left).  a = max |x| over the block; scale = 1 if a == 0,
    else binary32(a / QMAX); code = encode(binary32(x / scale)).
    """
    S = x.shape[0]
    qmax = _qmax(dtype)
    starts = np.arange(0, S, blk)
    a = np.maximum.reduceat(np.abs(x), starts, axis=0).max(axis=1)      # [nb]
    scale = np.where(a == 0, np.float32(1.0), a / qmax).astype(np.float32)
    per_tok = np.repeat(scale, blk)[:S]
    y = (x / per_tok[:, None]).astype(np.float32)
    return _encode(y, dtype), scale


MX_BLOCK = 32          # elements per MXFP8 scale block (along the head dimension)
MX_EMAX_E4M3 = 8       # exponent of the largest power of two E4M3 holds (448 = 1.75 * 2**8)


def _mx_quant_rows(x):
    """MXFP8 quantization of [S, D] binary32 rows in blocks of 32 channels.

    OCP Microscaling (MX) format with E4M3 elements and an E8M0 (power of
    two) shared scale per block: X = 2**(floor(log2(amax)) - 8), with 8 the
    exponent of E4M3's largest normal binade, clamped to E8M0's range
    [2**-127, 2**127] (2**-127 for an all-zero block); each element becomes
    E4M3(x / X), rounded to nearest even and saturated at 448 (amax / X lies
    in [256, 512)).  The division by a power of two is exact.
    Returns (codes uint8 [S, D], exponents int [S, D / 32]).
    """
    S, D = x.shape
    blocks = np.abs(x.astype(np.float64)).reshape(S, D // MX_BLOCK, MX_BLOCK)
    amax = blocks.max(axis=2)
    _, e = np.frexp(np.where(amax == 0, 1.0, amax))       # amax = m * 2**e, m in [0.5, 1)
    exp = np.where(amax == 0, -127, np.clip(e - 1 - MX_EMAX_E4M3, -127, 127))
    scale = np.ldexp(1.0, exp)
    y = x.astype(np.float64).reshape(S, D // MX_BLOCK, MX_BLOCK) / scale[:, :, None]
    return e4m3_encode(y.reshape(S, D)), exp.astype(np.int64)


def sage_quantize(q, k, v, qk_dtype, q_block, k_block, v_block=1, v_amax=None):
    """Quantization of Q, K and V for the low-precision attention recipes.

    The recipe is (qk_dtype, v_dtype = fp8, (q_block, k_block, v_block))
    ("VisualGen Quantized Attention", section "Recipes"):
      * SageAttention, qk_dtype int8 or fp8, blocks (1|4|16, 1|4|16, 1)
        ("SageAttention in the TRTLLM backend"): K-smoothing
        K_hat = binary32(K - mu) with mu from ``k_channel_mean``; Q and K_hat
        get one scale per block of ``q_block`` / ``k_block`` tokens per head.
      * QK16PV8, qk_dtype bf16, blocks (0, 0, 0) ("QK16PV8 Attention Kernels
        in the CUTEDSL Backend"): Q and K stay BF16 (no scales, no smoothing).
      * MXFP8 Q/K, qk_dtype mxfp8, blocks (0, 0, 0|1) ("MXFP8 and NVFP4 in
        the CUTEDSL and FlashInfer backends"): Q and K in OCP MXFP8, blocks
        of 32 channels along the head dimension (``_mx_quant_rows``); no
        smoothing (the pages tie smoothing to SageAttention only).
      * V: fp8 E4M3 with one scale per (batch, KV head, channel) for
        v_block = 1, or one tensor-wide scale for v_block = 0; scale =
        binary32(max|v| / 448) (1 if all zero).  ``v_amax`` supplies the
        tensor-wide max|v| for v_block = 0 when ``v`` holds only some heads
        of the tensor (it must be at least the slice's own maximum).

    Returns a dict: q_codes [B,Hq,S,D], k_codes [B,Hkv,S,D] (int8, uint8
    E4M3 bits, or float32 BF16 values), q_scale / k_scale (binary32 per token
    block [B,H,ceil(S/blk)] for SageAttention; E8M0 exponents [B,H,S,4] for
    MXFP8; absent for BF16), v_codes [B,Hkv,S,D] (uint8 E4M3), v_scale
    [B,Hkv,D] (binary32, all equal for v_block 0), mu [B,Hkv,D].
    """
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    B, Sq, Skv, Hq, Hkv, D = _shape_check(qf, kf, vf)
    sage = qk_dtype in ("int8", "fp8", "fp8_e4m3")
    if sage:
        if q_block < 1 or k_block < 1 or v_block != 1:
            raise ValueError(f"SageAttention blocks must be (>= 1, >= 1, 1), got {(q_block, k_block, v_block)}")
    elif qk_dtype == "bf16":
        if (q_block, k_block, v_block) != (0, 0, 0):
            raise ValueError("QK16PV8 takes blocks (0, 0, 0)")
    elif qk_dtype == "mxfp8":
        if (q_block, k_block) != (0, 0) or v_block not in (0, 1):
            raise ValueError("MXFP8 Q/K takes blocks (0, 0, 0) or (0, 0, 1)")
    else:
        raise ValueError(f"unsupported qk dtype {qk_dtype!r}")
    mu = k_channel_mean(kf) if sage else np.zeros((B, Hkv, D), np.float32)
    cdt = {"int8": np.int8, "bf16": np.float32}.get(qk_dtype, np.uint8)
    out = {
        "q_codes": np.empty((B, Hq, Sq, D), cdt),
        "k_codes": np.empty((B, Hkv, Skv, D), cdt),
        "v_codes": np.empty((B, Hkv, Skv, D), np.uint8),
        "v_scale": np.empty((B, Hkv, D), np.float32),
        "mu": mu,
        "qk_dtype": qk_dtype, "q_block": q_block, "k_block": k_block, "v_block": v_block,
    }
    if sage:
        out["q_scale"] = np.empty((B, Hq, -(-Sq // q_block)), np.float32)
        out["k_scale"] = np.empty((B, Hkv, -(-Skv // k_block)), np.float32)
    elif qk_dtype == "mxfp8":
        out["q_scale"] = np.empty((B, Hq, Sq, D // MX_BLOCK), np.int64)
        out["k_scale"] = np.empty((B, Hkv, Skv, D // MX_BLOCK), np.int64)
    for b in range(B):
        for h in range(Hq):
            if sage:
                out["q_codes"][b, h], out["q_scale"][b, h] = _block_quant_head(qf[b, :, h], q_block, qk_dtype)
            elif qk_dtype == "mxfp8":
                out["q_codes"][b, h], out["q_scale"][b, h] = _mx_quant_rows(qf[b, :, h])
            else:
                out["q_codes"][b, h] = qf[b, :, h]
        for g in range(Hkv):
            if sage:
                khat = (kf[b, :, g] - mu[b, g][None, :]).astype(np.float32)
                out["k_codes"][b, g], out["k_scale"][b, g] = _block_quant_head(khat, k_block, qk_dtype)
            elif qk_dtype == "mxfp8":
                out["k_codes"][b, g], out["k_scale"][b, g] = _mx_quant_rows(kf[b, :, g])
            else:
                out["k_codes"][b, g] = kf[b, :, g]
    vmax = np.float32(E4M3_MAX)
    if v_block == 0:
        if v_amax is not None:   # the tensor-wide maximum, when v is a slice (some heads) of the tensor
            a = np.float32(v_amax)
            if vf.size and np.abs(vf).max() > a:
                raise ValueError("v_amax is below the largest |v| of the slice")
        else:
            a = np.float32(np.abs(vf).max()) if vf.size else np.float32(0.0)
        out["v_scale"][...] = np.float32(1.0) if a == 0 else np.float32(a / vmax)
    else:
        a = np.abs(vf).max(axis=1)                                 # [B, Hkv, D]
        out["v_scale"][...] = np.where(a == 0, np.float32(1.0), a / vmax).astype(np.float32)
    for b in range(B):
        for g in range(Hkv):
            out["v_codes"][b, g] = e4m3_encode((vf[b, :, g] / out["v_scale"][b, g][None, :]).astype(np.float32))
    return out


def _logits(quant, b, h, g, rows, keys, sm_scale):
    """Logits s_ij = sm_scale * <dequantized q_i, dequantized k_j> (natural
    units) of one (batch, query head), from the codes and scales of
    ``sage_quantize``: sq(i) sk(j) <qc_i, kc_j> for SageAttention, the BF16
    dot for QK16PV8, and the sum over 32-channel blocks of X_q X_k <qc, kc>
    for MXFP8.  Every dot is exact in float64 (int8 sums stay below 2**21,
    products of E4M3 codes carry at most 8 significant bits)."""
    dt = quant["qk_dtype"]
    qc = _decode(quant["q_codes"][b, h][rows], dt)
    kc = _decode(quant["k_codes"][b, g][keys], dt)
    if dt == "bf16":
        dots = qc @ kc.T
    elif dt == "mxfp8":
        xq = np.ldexp(1.0, quant["q_scale"][b, h][rows])           # [R, 4]
        xk = np.ldexp(1.0, quant["k_scale"][b, g][keys])           # [N, 4]
        dots = np.zeros((len(rows), len(keys)))
        for blk in range(qc.shape[1] // MX_BLOCK):
            c = slice(MX_BLOCK * blk, MX_BLOCK * (blk + 1))
            dots += xq[:, blk][:, None] * xk[:, blk][None, :] * (qc[:, c] @ kc[:, c].T)
    else:
        sq = quant["q_scale"][b, h][rows // quant["q_block"]].astype(np.float64)
        sk = quant["k_scale"][b, g][keys // quant["k_block"]].astype(np.float64)
        dots = sq[:, None] * sk[None, :] * (qc @ kc.T)
    return sm_scale * dots


# How P enters BMM2.  The pages say only that both matmuls of SAGE run in low
# precision ("TRTLLM Attention", section "SAGE quantization"; "VisualGen
# Quantized Attention", section "Overview": BMM1 and BMM2 on narrower
# instructions), so P, BMM2's left operand, is FP8 E4M3 like V; they give
# neither P's scale, nor the reference it is taken against, nor how the row
# sum is formed.  Reading taken: the plain online softmax with only BMM2's
# operand narrowed.  The reference m is the exact running maximum of s over
# the tiles so far; p = exp(s - m) lies in (0, 1]; BMM2 multiplies
# p~ = E4M3(2**8 p) (2**8 keeps p's useful range inside E4M3's normal
# binades; at most 256 < 448, so nothing saturates); the row sum, a softmax
# statistic and not a matmul operand, adds the unrounded p.
def _sage_tile(m, l, acc, st, vt, quantize_p, p_scale):
    """One KV tile of the SAGE online softmax: logits ``st`` [R, n] and
    dequantized V codes ``vt`` [n, D].  State: running maximum m, row sum l
    (in units of p), accumulator acc (in units of p_scale * p times the V
    codes).  Returns the updated (m, l, acc)."""
    m2 = np.maximum(m, st.max(axis=1))
    alpha = np.where(np.isneginf(m), 0.0, np.exp(m - m2))
    p = np.exp(st - m2[:, None])
    pt = e4m3_decode(e4m3_encode(p_scale * p)) if quantize_p else p_scale * p
    return m2, alpha * l + p.sum(axis=1), alpha[:, None] * acc + pt @ vt


def sage_attention(quant, sm_scale, block_n, rows=None, quantize_p=True, p_scale=256.0,
                   out_dtype=None):
    """SAGE attention on quantized codes, emulated tile by tile in float64.

    Both matmuls run on low-precision operands ("TRTLLM Attention", section
    "SAGE quantization"; "VisualGen Quantized Attention", section
    "SageAttention in the TRTLLM backend").  Steps, for each query row i:
      * BMM1 and its scale: s_ij = sm_scale * sq(i) * sk(j) * <qc_i, kc_j>,
        the dot exact (int8 or E4M3 codes); for QK16PV8 the BF16 dot, for
        MXFP8 the sum over 32-channel blocks of X_q X_k <qc, kc> (``_logits``).
      * KV tiles of ``block_n`` keys in ascending order, each updating the
        online softmax state (``_sage_tile``): m' = max(m, tile max),
        alpha = exp(m - m') (0 while m = -inf), p_ij = exp(s_ij - m'),
        p~_ij = E4M3(2**8 p_ij) (``quantize_p``; 2**8 is ``p_scale``),
        l = alpha l + sum_j p_ij (the unrounded p),
        acc_d = alpha acc_d + sum_j p~_ij dec(vc_jd), m = m'.
      * Epilogue (the BMM2 scale): O_id = acc_d * sv_d / (2**8 l_i).
    With ``quantize_p`` off this is exact softmax attention on the
    dequantized tensors.  Returns O [B, R, Hq, D] (float64 unless
    ``out_dtype`` rounds it).
    """
    qc_all, kc_all, vc_all = quant["q_codes"], quant["k_codes"], quant["v_codes"]
    B, Hq, Sq, D = qc_all.shape
    Hkv, Skv = kc_all.shape[1], kc_all.shape[2]
    G = Hq // Hkv
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    R = len(rows)
    out = np.empty((B, R, Hq, D))
    keys = np.arange(Skv)
    for b in range(B):
        for g in range(Hkv):
            vd = e4m3_decode(vc_all[b, g])
            sv = quant["v_scale"][b, g].astype(np.float64)
            for h in range(g * G, (g + 1) * G):
                s = _logits(quant, b, h, g, rows, keys, sm_scale)
                m = np.full(R, -np.inf)
                l = np.zeros(R)
                acc = np.zeros((R, D))
                for t0 in range(0, Skv, block_n):
                    m, l, acc = _sage_tile(m, l, acc, s[:, t0:t0 + block_n], vd[t0:t0 + block_n],
                                           quantize_p, p_scale)
                out[b, :, h, :] = acc * sv[None, :] / (p_scale * l[:, None])
    return _round_out(out, out_dtype)


def sage_skip_attention(quant, sm_scale, factor, block_m, block_n, qtiles=None, quantize_p=True,
                        p_scale=256.0, out_dtype=None):
    """SAGE attention with the Skip-Softmax tile test, emulated in float64.

    Both options in one pass ("Diffusion Attention Backends" and "TRTLLM
    Attention": Skip-Softmax runs on the same TRTLLM backend as SAGE;
    "VisualGen Quantized Attention", section "Interaction With Other
    Features": the two are exercised together; "SAGE + Skip-Softmax - API
    Design & Test Plan", Part 1 section 4 for threshold = factor / seqlen).
    Readings taken:
      * the skip test runs on the dequantized logits of the SAGE path,
        s_ij = sm_scale * sq(i) * sk(j) * <qc_i, kc_j> (``_logits``);
      * queries in tiles of ``block_m`` rows, keys in the KV tiles of
        ``block_n`` keys of the SAGE online softmax; tile t > 0 of a query
        tile is skipped iff every valid row i has exp(M_it - m_i) < lambda =
        factor / S_kv, M_it the row's largest s in the tile and m_i its exact
        running maximum over the kept tiles;
      * a skipped tile changes nothing: not m, not the softmax reference, not
        the row sum, not the accumulator;
      * every kept tile is processed exactly as in ``sage_attention``.
    ``qtiles`` selects query tiles (default: all).  Returns (O [B, R, Hq, D],
    skipped [B, Hq, nQT, T] bool, ratio [B, Hq, nQT, T] = max_i
    exp(M_it - m_i) with NaN at t = 0, rows).
    """
    qc_all, kc_all, vc_all = quant["q_codes"], quant["k_codes"], quant["v_codes"]
    B, Hq, Sq, D = qc_all.shape
    Hkv, Skv = kc_all.shape[1], kc_all.shape[2]
    G = Hq // Hkv
    nqt = -(-Sq // block_m)
    T = -(-Skv // block_n)
    qtiles = np.arange(nqt) if qtiles is None else np.asarray(qtiles)
    lam = float(factor) / Skv
    ln_lam = math.log(lam) if lam > 0 else -math.inf
    rows = np.concatenate([np.arange(t * block_m, min(Sq, (t + 1) * block_m)) for t in qtiles])
    out = np.empty((B, len(rows), Hq, D))
    skipped = np.zeros((B, Hq, len(qtiles), T), bool)
    ratio = np.full((B, Hq, len(qtiles), T), np.nan)
    keys = np.arange(Skv)
    for b in range(B):
        for g in range(Hkv):
            vd = e4m3_decode(vc_all[b, g])
            sv = quant["v_scale"][b, g].astype(np.float64)
            for h in range(g * G, (g + 1) * G):
                r0 = 0
                for qi, qt in enumerate(qtiles):
                    rr = np.arange(qt * block_m, min(Sq, (qt + 1) * block_m))
                    s = _logits(quant, b, h, g, rr, keys, sm_scale)
                    m = np.full(len(rr), -np.inf)
                    l = np.zeros(len(rr))
                    acc = np.zeros((len(rr), D))
                    for t in range(T):
                        st = s[:, t * block_n:(t + 1) * block_n]
                        mt = st.max(axis=1)
                        if t > 0:
                            gap = mt - m
                            ratio[b, h, qi, t] = math.exp(gap.max())
                            if np.all(gap < ln_lam):
                                skipped[b, h, qi, t] = True
                                continue
                        m, l, acc = _sage_tile(m, l, acc, st, vd[t * block_n:(t + 1) * block_n],
                                               quantize_p, p_scale)
                    out[b, r0:r0 + len(rr), h, :] = acc * sv[None, :] / (p_scale * l[:, None])
                    r0 += len(rr)
    return _round_out(out, out_dtype), skipped, ratio, rows


# ----------------------------------------------------------------------------
# Skip-Softmax
# ----------------------------------------------------------------------------

def skip_attention(q, k, v, sm_scale, factor, block_m, block_n, qtiles=None, out_dtype=None, return_lse=False):
    """Skip-Softmax attention in float64, with its skipped-tile set.

    The pages define the threshold as factor / seqlen (the knob to
    kernel-argument table of "SAGE + Skip-Softmax - API Design & Test Plan",
    Part 1 section 4) and the effect as skipping low-contribution attention
    work ("TRTLLM Attention", section "Skip-Softmax"); the feature design doc
    with the exact rule is not among the pages.  Reading taken (seqlen =
    S_kv, tiles of ``block_m`` query rows x ``block_n`` keys):
      for each (batch, head, query tile) with running maxima m_i = -inf,
      KV tiles t = 0, 1, ... in order; M_it = max of s_ij over the tile;
      the tile is skipped iff t > 0 and, for every valid row i,
      exp(M_it - m_i) < lambda = factor / S_kv; otherwise m_i = max(m_i, M_it)
      and the tile's keys join row i's key set.  O_i is exact softmax
      attention over the kept keys only.
    ``qtiles`` selects query tiles (default: all).  Returns (O [B, R, Hq, D]
    for the rows of the selected tiles, skipped [B, Hq, nQT, T] bool,
    ratio [B, Hq, nQT, T] = max_i exp(M_it - m_i) with NaN at t = 0, rows),
    plus the LSE [B, Hq, R] over the kept keys with ``return_lse``.
    """
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    B, Sq, Skv, Hq, Hkv, D = _shape_check(qf, kf, vf)
    G = Hq // Hkv
    nqt = -(-Sq // block_m)
    T = -(-Skv // block_n)
    qtiles = np.arange(nqt) if qtiles is None else np.asarray(qtiles)
    lam = float(factor) / Skv
    ln_lam = math.log(lam) if lam > 0 else -math.inf
    rows = np.concatenate([np.arange(t * block_m, min(Sq, (t + 1) * block_m)) for t in qtiles])
    out = np.empty((B, len(rows), Hq, D))
    lse = np.empty((B, Hq, len(rows)))
    skipped = np.zeros((B, Hq, len(qtiles), T), bool)
    ratio = np.full((B, Hq, len(qtiles), T), np.nan)
    tile_starts = np.arange(0, Skv, block_n)
    tile_of_key = np.arange(Skv) // block_n
    for b in range(B):
        for h in range(Hq):
            kg, vg = kf[b, :, h // G, :], vf[b, :, h // G, :]
            r0 = 0
            for qi, qt in enumerate(qtiles):
                rr = np.arange(qt * block_m, min(Sq, (qt + 1) * block_m))
                s = sm_scale * (qf[b, rr, h, :] @ kg.T)                  # [r, S_kv]
                M = np.maximum.reduceat(s, tile_starts, axis=1)            # [r, T]
                m = np.full(len(rr), -np.inf)
                for t in range(T):
                    if t > 0:
                        gap = M[:, t] - m
                        ratio[b, h, qi, t] = math.exp(gap.max())
                        if np.all(gap < ln_lam):
                            skipped[b, h, qi, t] = True
                            continue
                    m = np.maximum(m, M[:, t])
                keep = ~skipped[b, h, qi][tile_of_key]                     # [S_kv]
                sk = np.where(keep[None, :], s, -np.inf)
                mx = sk.max(axis=1, keepdims=True)
                p = np.exp(sk - mx)
                l = p.sum(axis=1, keepdims=True)
                out[b, r0:r0 + len(rr), h, :] = (p @ vg) / l
                lse[b, h, r0:r0 + len(rr)] = (mx + np.log(l))[:, 0]
                r0 += len(rr)
    res = (_round_out(out, out_dtype), skipped, ratio, rows)
    return res + (lse,) if return_lse else res


def skip_gate_enabled(t, D):
    """Host-side timestep gate: Skip-Softmax is on for a step iff t <= D.

    t is the normalized denoising timestep, running from 1 (noisiest) to 0;
    both values must be finite and in [0, 1] ("TRTLLM Attention", section
    "Skip-Softmax", key disabled_until_timestep; the design doc's knob table
    calls it a host-side gate with no kernel argument).
    """
    vals = []
    for name, x in (("t", t), ("D", D)):
        try:
            xf = float(x)
        except (TypeError, ValueError):
            raise ValueError(f"{name} must be a real number, got {x!r}") from None
        if not (math.isfinite(xf) and 0.0 <= xf <= 1.0):
            raise ValueError(f"{name} must be finite and in [0, 1], got {x!r}")
        vals.append(xf)
    return vals[0] <= vals[1]

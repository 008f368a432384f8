"""Seeded synthetic inputs shaped like diffusion-transformer attention.

This module only draws random tensors and lays them out; it holds none of the
attention method's arithmetic, so both the CPU oracle's tests and the HIP
path's tests and benchmark can take their inputs from it.

Every tensor is drawn in float32 from ``numpy.random.Generator(PCG64(seed))``
in a fixed order and rounded to bfloat16 (round-to-nearest-even, by torch's
conversion).  Layout is ``[B, S, H, D]`` with ``D`` contiguous, as the
"packed, mask-free" layout of the TRTLLM Attention page (section
"Requirements") describes.

Workloads (``WORKLOADS``) mirror the shapes the pages run on: Wan 2.2 video
(token grid 21 x 45 x 80 = 75,600, 40 heads, head_dim 128), plus a GQA and a
small case.  No dataset, prompt or checkpoint is involved.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

HEAD_DIM = 128
WAN_GRID = (21, 45, 80)  # frames x rows x cols of a Wan-shaped latent video


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "dense", "sage", "skip"
    B: int
    S: int
    Hq: int
    Hkv: int
    gen: str             # "gauss" or "positional"
    k_bias_std: float = 0.0
    outliers: int = 0
    out_dtype: str = "bf16"
    recipe: tuple | None = None       # (qk_dtype, v_dtype, (qb, kb, vb))
    factors: tuple = field(default=())  # skip threshold factors
    grid: tuple | None = None


WORKLOADS = {
    w.name: w
    for w in (
        Workload("dense_b1_h2_s256", "dense", 1, 256, 2, 2, "gauss", out_dtype="fp32"),
        Workload("dense_gqa_b2_h24kv8_s8192", "dense", 2, 8192, 24, 8, "gauss", k_bias_std=2.0),
        Workload("sage_int8_b1_h40_s32768", "sage", 1, 32768, 40, 40, "gauss",
                 k_bias_std=4.0, outliers=4, recipe=("int8", "fp8", (1, 16, 1))),
        Workload("sage_fp8_wan_b1_h40_s75600", "sage", 1, 75600, 40, 40, "gauss",
                 k_bias_std=4.0, outliers=4, recipe=("fp8", "fp8", (1, 4, 1))),
        Workload("skip_wan_b1_h40_s75600", "skip", 1, 75600, 40, 40, "positional",
                 factors=(0.0, 1.0, 10.0, 100.0), grid=WAN_GRID),
    )
}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def gaussian_qkv(B, S, Hq, Hkv, D=HEAD_DIM, seed=0, k_bias_std=0.0, outliers=0,
                 outlier_mult=8.0, std=1.0):
    """Q, V ~ N(0, std); K ~ N(0, std) + bias[h, d].

    The bias is one value per (KV head, channel), shared by every token and
    batch entry, drawn N(0, k_bias_std) (second argument = standard
    deviation).  ``outliers`` channel indices, the same for every head, get
    their bias multiplied by ``outlier_mult``.  Draw order: Q, K, V, bias,
    outlier indices.
    """
    rng = _rng(seed)
    q = _to_bf16(rng.standard_normal((B, S, Hq, D), dtype=np.float32) * np.float32(std))
    kf = rng.standard_normal((B, S, Hkv, D), dtype=np.float32) * np.float32(std)
    v = _to_bf16(rng.standard_normal((B, S, Hkv, D), dtype=np.float32) * np.float32(std))
    if k_bias_std > 0.0:
        bias = rng.standard_normal((Hkv, D), dtype=np.float32) * np.float32(k_bias_std)
        if outliers:
            idx = rng.choice(D, size=outliers, replace=False)
            bias[:, idx] *= np.float32(outlier_mult)
        kf += bias[None, None, :, :]
    k = _to_bf16(kf)
    del kf
    return q, k, v


def position_code(grid, D=HEAD_DIM):
    """3-D sinusoidal code of token n -> (frame, row, col), float64 [S, D].

    n maps to (n // (R*C), (n // C) % R, n % C).  The D/2 (cos, sin) pairs are
    split over the axes as 22, 21, 21 (for D = 128); pair k of axis a uses the
    angular frequency pi * L_a ** (-k / K_a), with L_a the axis length and K_a
    its pair count.
    """
    F, R, C = grid
    S = F * R * C
    n = np.arange(S)
    coords = (n // (R * C), (n // C) % R, n % C)
    pairs = D // 2
    split = [pairs - 2 * (pairs // 3), pairs // 3, pairs // 3]
    cols = []
    for x, L, K in zip(coords, grid, split):
        for kk in range(K):
            w = math.pi * float(L) ** (-kk / K)
            cols.append(np.cos(w * x))
            cols.append(np.sin(w * x))
    return np.stack(cols, axis=1)


def positional_qkv(grid=WAN_GRID, H=40, D=HEAD_DIM, seed=0, noise=0.5, alpha=1.456, B=1):
    """Spatially peaked Q/K: 0.5 * N(0,1) + alpha * R_h c(n); V ~ N(0,1).

    c(n) is ``position_code``; R_h is a per-head orthogonal matrix (QR of a
    Gaussian matrix with the signs of R's diagonal folded in), the stand-in
    for the learned projection.  With alpha = 1.456 the self logit sits about
    12 above the far field at scale 1/sqrt(128).  Draw order: Q noise, K
    noise, V, then the H Gaussian matrices.
    """
    S = grid[0] * grid[1] * grid[2]
    rng = _rng(seed)
    qn = rng.standard_normal((B, S, H, D), dtype=np.float32) * np.float32(noise)
    kn = rng.standard_normal((B, S, H, D), dtype=np.float32) * np.float32(noise)
    v = _to_bf16(rng.standard_normal((B, S, H, D), dtype=np.float32))
    code = position_code(grid, D)
    for h in range(H):
        g = rng.standard_normal((D, D))
        qm, rm = np.linalg.qr(g)
        qm = qm * np.sign(np.diag(rm))[None, :]
        proj = (alpha * (code @ qm.T)).astype(np.float32)
        qn[:, :, h, :] += proj[None]
        kn[:, :, h, :] += proj[None]
    q = _to_bf16(qn)
    del qn
    k = _to_bf16(kn)
    del kn
    return q, k, v


def generate(name: str, seed: int = 0, S: int | None = None, H: int | None = None):
    """Inputs of a named workload, optionally with fewer tokens or heads.

    A smaller ``S`` keeps the value distribution of the workload (for the
    positional generator the grid is cut to whole frames when it can be, else
    to a 1 x 1 x S line).  Returns (q, k, v) as CPU bfloat16 tensors.
    """
    w = WORKLOADS[name]
    S = w.S if S is None else S
    Hq = w.Hq if H is None else H
    Hkv = w.Hkv if H is None else max(1, H * w.Hkv // w.Hq)
    if w.gen == "gauss":
        return gaussian_qkv(w.B, S, Hq, Hkv, seed=seed, k_bias_std=w.k_bias_std,
                            outliers=w.outliers)
    grid = w.grid
    if S != grid[0] * grid[1] * grid[2]:
        per_frame = grid[1] * grid[2]
        grid = (S // per_frame, grid[1], grid[2]) if S % per_frame == 0 else (1, 1, S)
    return positional_qkv(grid, H=Hq, seed=seed, B=w.B)


def attention_flops(B, S_q, S_kv, Hq, D=HEAD_DIM):
    """Effective work of one attention call: 4 * B * Hq * S_q * S_kv * D."""
    return 4.0 * B * Hq * S_q * S_kv * D

"""Seeded synthetic inputs shaped like diffusion-transformer attention.

This module only draws random tensors and lays them out; it holds none of the
attention method's arithmetic, so both the CPU oracle's tests and the HIP
path's tests and benchmark take their inputs from it.

Random draws come from torch's counter-based generator (Philox on a GPU,
torch's CPU generator on the host) seeded with ``seed``, in float32, in a
fixed order, then rounded to bfloat16 (round-to-nearest-even, torch's
conversion).  The same seed, shape and device give the same tensors on every
run; a test generates once and hands the very same tensor to the HIP path and
to the oracle.  Large inputs are drawn on the GPU (``device="cuda"``) so that
Wan-sized tensors take seconds, not minutes.

Layout is ``[B, S, H, D]`` with ``D`` contiguous, the packed, mask-free layout
of the "TRTLLM Attention" page (section "Requirements").  Workloads
(``WORKLOADS``) mirror the shapes the pages run on: Wan 2.2 video (token grid
21 x 45 x 80 = 75,600, 40 heads, head_dim 128), a GQA case and a small case.
No dataset, prompt or checkpoint is involved.
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


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device, std=1.0):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def gaussian_qkv(B, S, Hq, Hkv, D=HEAD_DIM, seed=0, k_bias_std=0.0, outliers=0,
                 outlier_mult=8.0, std=1.0, device="cpu"):
    """Q, V ~ N(0, std); K ~ N(0, std) + bias[h, d]; bfloat16 [B, S, H, D].

    The bias is one value per (KV head, channel), shared by every token and
    batch entry, drawn N(0, k_bias_std) (second argument = standard
    deviation).  ``outliers`` channel indices, the same for every head, get
    their bias multiplied by ``outlier_mult``.  Draw order on the device
    generator: Q, K, V; the bias and the outlier indices come from a host
    generator seeded with seed + 1.
    """
    g = _gen(seed, device)
    q = _randn((B, S, Hq, D), g, device, std).to(torch.bfloat16)
    kf = _randn((B, S, Hkv, D), g, device, std)
    v = _randn((B, S, Hkv, D), g, device, std).to(torch.bfloat16)
    if k_bias_std > 0.0:
        rng = np.random.Generator(np.random.PCG64(seed + 1))
        bias = rng.standard_normal((Hkv, D)).astype(np.float32) * np.float32(k_bias_std)
        if outliers:
            idx = rng.choice(D, size=outliers, replace=False)
            bias[:, idx] *= np.float32(outlier_mult)
        kf += torch.from_numpy(bias).to(kf.device)[None, None]
    k = kf.to(torch.bfloat16)
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


def head_rotations(H, D=HEAD_DIM, seed=0):
    """Per-head orthogonal matrices: QR of a Gaussian matrix, signs fixed by R's diagonal."""
    rng = np.random.Generator(np.random.PCG64(seed + 2))
    out = np.empty((H, D, D))
    for h in range(H):
        qm, rm = np.linalg.qr(rng.standard_normal((D, D)))
        out[h] = qm * np.sign(np.diag(rm))[None, :]
    return out


def positional_qkv(grid=WAN_GRID, H=40, D=HEAD_DIM, seed=0, noise=0.5, alpha=1.456, B=1, device="cpu"):
    """Spatially peaked Q/K: noise * N(0,1) + alpha * R_h c(n); V ~ N(0,1).

    c(n) is ``position_code``; R_h (``head_rotations``) is the per-head
    stand-in for the learned projection.  With alpha = 1.456 the self logit
    sits about 12 above the far field at scale 1/sqrt(128).  Draw order on the
    device generator: Q noise, K noise, V; the projection is added in float64
    and the sum rounded to float32, then to bfloat16.
    """
    S = grid[0] * grid[1] * grid[2]
    g = _gen(seed, device)
    qn = _randn((B, S, H, D), g, device, noise)
    kn = _randn((B, S, H, D), g, device, noise)
    v = _randn((B, S, H, D), g, device).to(torch.bfloat16)
    code = torch.from_numpy(position_code(grid, D)).to(device)
    rot = torch.from_numpy(head_rotations(H, D, seed)).to(device)
    for h in range(H):
        proj = (alpha * (code @ rot[h].T)).to(torch.float32)
        qn[:, :, h, :] += proj[None]
        kn[:, :, h, :] += proj[None]
    q = qn.to(torch.bfloat16)
    del qn
    k = kn.to(torch.bfloat16)
    del kn
    return q, k, v


def generate(name: str, seed: int = 0, S: int | None = None, H: int | None = None, device="cpu"):
    """Inputs of a named workload, optionally with fewer tokens or heads.

    A smaller ``S`` keeps the value distribution of the workload (for the
    positional generator the grid is cut to whole frames when it can be, else
    to a 1 x 1 x S line).  Returns (q, k, v) bfloat16 tensors on ``device``.
    """
    w = WORKLOADS[name]
    S = w.S if S is None else S
    Hq = w.Hq if H is None else H
    Hkv = w.Hkv if H is None else max(1, H * w.Hkv // w.Hq)
    if w.gen == "gauss":
        return gaussian_qkv(w.B, S, Hq, Hkv, seed=seed, k_bias_std=w.k_bias_std,
                            outliers=w.outliers, device=device)
    grid = w.grid
    if S != grid[0] * grid[1] * grid[2]:
        per_frame = grid[1] * grid[2]
        grid = (S // per_frame, grid[1], grid[2]) if S % per_frame == 0 else (1, 1, S)
    return positional_qkv(grid, H=Hq, seed=seed, B=w.B, device=device)


def attention_flops(B, S_q, S_kv, Hq, D=HEAD_DIM):
    """Effective work of one attention call: 4 * B * Hq * S_q * S_kv * D."""
    return 4.0 * B * Hq * S_q * S_kv * D

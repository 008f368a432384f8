"""Helpers shared by the GPU parity tests (comparison metrics, device checks)."""
import math
import os
import sys

import numpy as np
import pytest
import torch

gpu_available = torch.cuda.is_available()
needs_gpu = pytest.mark.skipif(not gpu_available, reason="needs an MI355X GPU")


def announce(msg):
    """Name the case on stdout before a GPU step, so a failing run says which."""
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def dense_tolerances(got, ref):
    """Dense BF16 parity bar: max-abs <= 1e-2 and rel-L2 <= 5e-3."""
    ma, rl = max_abs(got, ref), rel_l2(got, ref)
    assert ma <= 1e-2 and rl <= 5e-3, f"max_abs={ma:.3e} rel_l2={rl:.3e}"
    return ma, rl


def ramp_qkv(S, step, seed, sign=1.0):
    """Logits that change by `step` (natural units, sm_scale 1/sqrt(128) folded in) per key in
    key order, on top of Gaussian noise: with a rising ramp every KV tile raises the row
    maximum, so the running reference moves and the accumulators are rescaled again and again."""
    g = torch.Generator().manual_seed(seed)
    q = 0.3 * torch.randn(1, S, 2, 128, generator=g)
    k = 0.3 * torch.randn(1, S, 1, 128, generator=g)
    v = torch.randn(1, S, 1, 128, generator=g)
    q[..., 0] = 1.0
    k[0, :, 0, 0] = sign * step * math.sqrt(128) * torch.arange(S, dtype=torch.float32)
    return q.bfloat16(), k.bfloat16(), v.bfloat16()


def compare_skip_sets(got, ref_skip, ratio, lam, log_band, label=""):
    """Skipped-tile sets must be identical except on tiles whose decision sits
    within the tie band of the threshold: |ln(ratio) - ln(lambda)| <= max(1e-6,
    log_band), with ratio = max_i exp(M_it - m_i) from the oracle.  The 1e-6 is
    the tie band read on the natural-log logit difference; ``log_band`` widens it
    to the rounding bound of the kernel's own logits.  Prints the band and flip
    counts and asserts that every flip lies inside the band."""
    with np.errstate(divide="ignore", invalid="ignore"):
        dist = np.abs(np.log(ratio) - math.log(lam))
    near = (dist <= max(1e-6, log_band)) & ~np.isnan(ratio)
    flips = got != ref_skip
    outside = flips & ~near
    sys.stdout.write(f"[skip-set] {label} tiles={flips.size} skipped={int(ref_skip.sum())} band={int(near.sum())} "
                     f"flips={int(flips.sum())}\n")
    assert not outside.any(), f"{int(outside.sum())} tiles differ outside the band (band tiles: {int(near.sum())})"
    return int(near.sum()), int(flips.sum())


def parallel_map(fn, items):
    """Map ``fn`` over ``items`` on threads (the oracle's numpy work releases the
    GIL), at most 16 at a time."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        return list(ex.map(fn, items))


def sample_tiles(n_tiles, count, seed=0):
    """``count`` distinct tile indices out of ``n_tiles``: the first, the last
    (often partial) and a seeded spread in between."""
    inner = np.random.default_rng(seed).choice(np.arange(1, n_tiles - 1), size=count - 2, replace=False)
    return np.unique(np.concatenate([[0, n_tiles - 1], inner]))

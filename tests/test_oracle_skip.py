"""Pins of the oracle's Skip-Softmax emulation and the host timestep gate."""
import math

import numpy as np
import pytest

from oracle import exact_attention, skip_attention, skip_gate_enabled
from diffusion_transformer_attention_non_amd.synth import positional_qkv

SC = 1 / math.sqrt(128)


@pytest.fixture(scope="module")
def peaked():
    q, k, v = positional_qkv(grid=(2, 8, 24), H=2, seed=3)
    return q.double().numpy(), k.double().numpy(), v.double().numpy()


def test_factor_zero_is_exact_attention(peaked):
    q, k, v = peaked
    o, skipped, _, rows = skip_attention(q, k, v, SC, 0.0, 32, 32)
    assert not skipped.any()
    np.testing.assert_allclose(o, exact_attention(q, k, v, SC, rows=rows), rtol=0, atol=1e-13)


def test_skip_sets_are_monotone_in_factor_and_never_first_tile(peaked):
    q, k, v = peaked
    prev = None
    fracs = []
    for f in (0.5, 1.0, 10.0, 100.0):
        _, sk, _, _ = skip_attention(q, k, v, SC, f, 32, 32)
        assert not sk[..., 0].any()
        if prev is not None:
            assert np.all(sk >= prev)
        prev = sk
        fracs.append(sk.mean())
    assert fracs[-1] > 0.3 and fracs[0] < fracs[-1]


def _brute_skip(q, k, v, sc, factor, bm, bn):
    """Scalar loops: tile maxima, running maxima, skip vote, restricted softmax."""
    B, S, Hq, D = q.shape
    lam = factor / S
    T = -(-S // bn)
    out = np.zeros_like(q)
    skip = np.zeros((B, Hq, -(-S // bm), T), bool)
    for b in range(B):
        for h in range(Hq):
            for qt in range(-(-S // bm)):
                rows = range(qt * bm, min(S, qt * bm + bm))
                s = {i: [sc * math.fsum(q[b, i, h, d] * k[b, j, h, d] for d in range(D)) for j in range(S)] for i in rows}
                m = {i: -math.inf for i in rows}
                kept = []
                for t in range(T):
                    keys = range(t * bn, min(S, t * bn + bn))
                    tmax = {i: max(s[i][j] for j in keys) for i in rows}
                    if t > 0 and all(math.exp(tmax[i] - m[i]) < lam for i in rows):
                        skip[b, h, qt, t] = True
                        continue
                    for i in rows:
                        m[i] = max(m[i], tmax[i])
                    kept.extend(keys)
                for i in rows:
                    mx = max(s[i][j] for j in kept)
                    p = {j: math.exp(s[i][j] - mx) for j in kept}
                    l = math.fsum(p.values())
                    for d in range(D):
                        out[b, i, h, d] = math.fsum(p[j] * v[b, j, h, d] for j in kept) / l
    return out, skip


def test_matches_scalar_brute_force_on_tiny_grid():
    q, k, v = positional_qkv(grid=(1, 4, 9), H=2, D=16, seed=4, alpha=2.2)
    q, k, v = q.double().numpy(), k.double().numpy(), v.double().numpy()
    sc = 0.25
    for factor in (0.0, 1.0, 4.0):
        o, sk, _, rows = skip_attention(q, k, v, sc, factor, 4, 4)
        ob, skb = _brute_skip(q, k, v, sc, factor, 4, 4)
        assert np.array_equal(sk, skb)
        np.testing.assert_allclose(o, ob[:, rows], rtol=0, atol=1e-13)
        if factor == 4.0:
            assert sk.any()


def test_dropped_mass_bound(peaked):
    q, k, v = peaked
    S = q.shape[1]
    dense, probs = exact_attention(q, k, v, SC, return_probs=True)
    o, sk, _, rows = skip_attention(q, k, v, SC, 100.0, 32, 32)
    vmax = np.abs(v).max()
    for h in range(2):
        keymask = np.repeat(sk[0, h], 32, axis=1)[:, :S]              # [nQT, S]
        dropped = (probs[0, h] * np.repeat(keymask, 32, axis=0)[:S]).sum(axis=1)
        err = np.abs(o[0, :, h] - dense[0, rows, h]).max(axis=1)
        assert np.all(err <= 2 * dropped / (1 - dropped) * vmax + 1e-13)


def test_every_later_tile_skipped_when_maxima_fall():
    S, D, bn = 64, 128, 16
    k = np.zeros((1, S, 1, D))
    q = np.zeros((1, S, 1, D))
    q[0, :, 0, 0] = 1.0
    # tile t's logits are -3t: each tile's maximum sits 3 below the previous one,
    # and exp(-3) < lambda = 4/64 < 1
    k[0, :, 0, 0] = -3.0 * (np.arange(S) // bn)
    v = np.random.default_rng(0).standard_normal((1, S, 1, D))
    o, sk, _, rows = skip_attention(q, k, v, 1.0, 4.0, 16, bn)
    assert sk[..., 1:].all() and not sk[..., 0].any()
    np.testing.assert_allclose(o[0, :, 0], np.broadcast_to(v[0, :bn, 0].mean(axis=0), (S, D)), rtol=0, atol=1e-14)


def test_selected_query_tiles_match_full_run(peaked):
    q, k, v = peaked
    o_all, sk_all, r_all, rows_all = skip_attention(q, k, v, SC, 10.0, 32, 32)
    sel = np.array([0, 5, 11])
    o, sk, r, rows = skip_attention(q, k, v, SC, 10.0, 32, 32, qtiles=sel)
    assert np.array_equal(sk, sk_all[:, :, sel])
    np.testing.assert_allclose(o, o_all[:, np.concatenate([np.arange(t * 32, t * 32 + 32) for t in sel])], atol=0, rtol=0)


@pytest.mark.parametrize("t,D,on", [(1.0, 1.0, True), (0.5, 0.5, True), (0.86, 0.86, True), (0.9, 0.86, False),
                                    (0.0, 0.0, True), (0.01, 0.0, False), (1.0, 0.99, False), (0.0, 1.0, True)])
def test_gate_truth_table(t, D, on):
    assert skip_gate_enabled(t, D) is on


@pytest.mark.parametrize("t,D", [(1.5, 0.5), (-0.1, 0.5), (0.5, float("nan")), (0.5, float("inf")), (0.5, "x")])
def test_gate_rejects_bad_values(t, D):
    with pytest.raises(ValueError):
        skip_gate_enabled(t, D)


def test_lse_factor_zero_and_kept_key_set(peaked):
    q, k, v = peaked
    _, _, _, rows, lse0 = skip_attention(q, k, v, SC, 0.0, 32, 32, return_lse=True)
    _, lse_exact = exact_attention(q, k, v, SC, rows=rows, return_lse=True)
    np.testing.assert_allclose(lse0, lse_exact, rtol=0, atol=1e-12)
    # with skipping, the LSE is that of exact attention over the kept keys of each query tile
    _, sk, _, rows, lse = skip_attention(q, k, v, SC, 100.0, 32, 32, qtiles=[3], return_lse=True)
    keep = ~sk[0, :, 0]                              # [Hq, T]
    for h in range(q.shape[2]):
        keys = np.flatnonzero(np.repeat(keep[h], 32)[:k.shape[1]])
        _, ref = exact_attention(q[:, :, h:h + 1], k[:, keys, h:h + 1], v[:, keys, h:h + 1], SC, rows=rows,
                                 return_lse=True)
        np.testing.assert_allclose(lse[0, h], ref[0, 0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("delta,skipped", [(-0.01, True), (0.01, False)])
def test_threshold_boundary_is_factor_over_seqlen_in_natural_log(delta, skipped):
    """Tile 1's maximum sits ln(lambda) + delta below tile 0's, lambda = factor / S_kv = 4 / 64
    ("threshold = factor / seqlen"; the tile is dropped when exp(M - m) < lambda).  A threshold
    without the division by S_kv, or taken in log2 units, puts both cases on the same side."""
    S, D, bn = 64, 128, 32
    lam = 4.0 / S
    q = np.zeros((1, S, 1, D))
    k = np.zeros((1, S, 1, D))
    q[0, :, 0, 0] = 1.0
    k[0, bn:, 0, 0] = math.log(lam) + delta
    v = np.random.default_rng(1).standard_normal((1, S, 1, D))
    _, sk, _, _ = skip_attention(q, k, v, 1.0, 4.0, 64, bn)
    assert not sk[..., 0].any()
    assert bool(sk[0, 0, 0, 1]) == skipped

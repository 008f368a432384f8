"""Pins of the oracle's exact attention: brute force, torch SDPA in float64,
closed forms and invariants."""
import math

import numpy as np
import pytest
import torch

from oracle import exact_attention


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _brute(q, k, v, sm_scale):
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Sq, Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(Sq):
                s = [sm_scale * math.fsum(q[b, i, h, d] * k[b, j, g, d] for d in range(D)) for j in range(Skv)]
                mx = max(s)
                p = [math.exp(x - mx) for x in s]
                l = math.fsum(p)
                for d in range(D):
                    out[b, i, h, d] = math.fsum(p[j] * v[b, j, g, d] for j in range(Skv)) / l
    return out


@pytest.mark.parametrize("S,Hq,Hkv", [(1, 1, 1), (2, 2, 1), (3, 1, 1), (5, 6, 2), (17, 2, 2)])
def test_exact_matches_brute_force(S, Hq, Hkv):
    D = 16 if S > 5 else 128
    q, k, v = _rand((2, S, Hq, D), 1), _rand((2, S, Hkv, D), 2), _rand((2, S, Hkv, D), 3)
    sc = 1 / math.sqrt(D)
    np.testing.assert_allclose(exact_attention(q, k, v, sc), _brute(q, k, v, sc), rtol=0, atol=1e-13)


@pytest.mark.parametrize("S,Hq,Hkv", [(130, 6, 2), (257, 4, 4), (64, 8, 1)])
def test_exact_matches_torch_sdpa_float64(S, Hq, Hkv):
    D = 128
    q, k, v = _rand((2, S, Hq, D), 4), _rand((2, S + 3, Hkv, D), 5, 2.0), _rand((2, S + 3, Hkv, D), 6)
    sc = 1 / math.sqrt(D)
    G = Hq // Hkv
    tq = torch.from_numpy(q).transpose(1, 2)
    tk = torch.from_numpy(k).repeat_interleave(G, dim=2).transpose(1, 2)
    tv = torch.from_numpy(v).repeat_interleave(G, dim=2).transpose(1, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=sc).transpose(1, 2).numpy()
    np.testing.assert_allclose(exact_attention(q, k, v, sc), ref, rtol=0, atol=1e-12)


def test_rows_of_p_sum_to_one_and_rows_subset():
    q, k, v = _rand((1, 40, 2, 128), 7, 3.0), _rand((1, 50, 2, 128), 8), _rand((1, 50, 2, 128), 9)
    o, p = exact_attention(q, k, v, 0.1, return_probs=True)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-13)
    rows = np.array([0, 13, 39])
    np.testing.assert_allclose(exact_attention(q, k, v, 0.1, rows=rows), o[:, rows], rtol=0, atol=1e-14)


def test_constant_v_returns_v():
    q, k = _rand((1, 33, 3, 128), 10, 4.0), _rand((1, 70, 3, 128), 11, 4.0)
    row = _rand((128,), 12)
    v = np.broadcast_to(row, (1, 70, 3, 128)).copy()
    o = exact_attention(q, k, v, 1 / math.sqrt(128))
    np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), rtol=1e-14, atol=1e-15)


def test_zero_q_gives_mean_of_v():
    k, v = _rand((1, 45, 2, 128), 13), _rand((1, 45, 2, 128), 14)
    q = np.zeros((1, 5, 2, 128))
    o = exact_attention(q, k, v, 0.3)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), rtol=0, atol=1e-14)


def test_one_dominant_key_returns_its_value_row():
    S, D = 20, 128
    k = _rand((1, S, 1, D), 15) * 1e-3
    q = np.zeros((1, 1, 1, D))
    q[0, 0, 0, 0] = 1.0
    k[0, 7, 0, 0] = 900.0                  # logit gap >= 800 -> exp(-gap) underflows to 0
    v = _rand((1, S, 1, D), 16)
    o = exact_attention(q, k, v, 1.0)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 7, 0])


def test_non_causal_permutation_equivariance():
    q, k, v = _rand((1, 31, 2, 128), 17), _rand((1, 29, 1, 128), 18), _rand((1, 29, 1, 128), 19)
    o = exact_attention(q, k, v, 0.09)
    pk = np.random.default_rng(0).permutation(29)
    np.testing.assert_allclose(exact_attention(q, k[:, pk], v[:, pk], 0.09), o, rtol=0, atol=1e-14)
    pq = np.random.default_rng(1).permutation(31)
    np.testing.assert_allclose(exact_attention(q[:, pq], k, v, 0.09), o[:, pq], rtol=0, atol=1e-15)


def test_gqa_group_shares_kv_head():
    # query heads 0..2 read KV head 0 and 3..5 read KV head 1 (consecutive grouping)
    q = _rand((1, 9, 6, 128), 20)
    k, v = _rand((1, 11, 2, 128), 21), _rand((1, 11, 2, 128), 22)
    o = exact_attention(q, k, v, 0.1)
    for h in range(6):
        g = h // 3
        oh = exact_attention(q[:, :, h:h + 1], k[:, :, g:g + 1], v[:, :, g:g + 1], 0.1)
        np.testing.assert_allclose(o[:, :, h:h + 1], oh, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- LSE

@pytest.mark.parametrize("Sq,Skv,Hq,Hkv", [(5, 9, 2, 1), (33, 17, 4, 2)])
def test_lse_matches_scipy_logsumexp(Sq, Skv, Hq, Hkv):
    from scipy.special import logsumexp
    rng = np.random.default_rng(21)
    q = rng.standard_normal((1, Sq, Hq, 128)) * 2
    k = rng.standard_normal((1, Skv, Hkv, 128)) * 2
    v = rng.standard_normal((1, Skv, Hkv, 128))
    _, lse = exact_attention(q, k, v, 0.3, return_lse=True)
    G = Hq // Hkv
    for h in range(Hq):
        logits = 0.3 * np.einsum("id,jd->ij", q[0, :, h], k[0, :, h // G])
        np.testing.assert_allclose(lse[0, h], logsumexp(logits, axis=1), rtol=0, atol=1e-12)


def test_lse_zero_q_is_log_of_key_count():
    rng = np.random.default_rng(22)
    k = rng.standard_normal((2, 37, 1, 128))
    v = rng.standard_normal((2, 37, 1, 128))
    _, lse = exact_attention(np.zeros((2, 5, 3, 128)), k, v, 0.1, return_lse=True)
    np.testing.assert_allclose(lse, np.full((2, 3, 5), math.log(37)), rtol=0, atol=1e-13)


def test_lse_merges_partial_results_over_key_subsets():
    """The property LSE is exported for: attention over keys A u B equals the
    LSE-weighted merge of the results over A and over B."""
    rng = np.random.default_rng(23)
    q = rng.standard_normal((1, 7, 1, 128))
    k = rng.standard_normal((1, 40, 1, 128))
    v = rng.standard_normal((1, 40, 1, 128))
    o, lse = exact_attention(q, k, v, 0.2, return_lse=True)
    oa, la = exact_attention(q, k[:, :13], v[:, :13], 0.2, return_lse=True)
    ob, lb = exact_attention(q, k[:, 13:], v[:, 13:], 0.2, return_lse=True)
    wa, wb = np.exp(la - lse)[0, 0], np.exp(lb - lse)[0, 0]
    np.testing.assert_allclose(wa + wb, 1.0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(o[0, :, 0], wa[:, None] * oa[0, :, 0] + wb[:, None] * ob[0, :, 0], rtol=0, atol=1e-13)

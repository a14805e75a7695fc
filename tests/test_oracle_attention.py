"""Pins of the oracle's decode and verify attention: closed forms, GQA head map,
torch's scaled_dot_product_attention (an independent library routine), causality,
and the two verify formulations against each other."""
import numpy as np
import pytest
import torch

from oracle import attention as A


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(0)
    q, K, V = _rand(rng, 4, 16), _rand(rng, 2, 1, 16), _rand(rng, 2, 1, 16)
    o, lse = A.decode(q, K, V, 0.25)
    for h in range(4):
        g = h // 2
        assert np.allclose(o[h], V[g, 0], atol=1e-14, rtol=0)
        assert np.isclose(lse[h], 0.25 * q[h] @ K[g, 0], atol=1e-13)


def test_equal_keys_give_mean_value_and_log_n():
    rng = np.random.default_rng(1)
    n, d = 50, 8
    K = np.repeat(_rand(rng, 1, 1, d), n, axis=1)
    V = _rand(rng, 1, n, d)
    q = _rand(rng, 3, d)
    o, lse = A.decode(q, K, V, 0.5)
    for h in range(3):
        assert np.allclose(o[h], V[0].mean(axis=0), atol=1e-13)
        assert np.isclose(lse[h], 0.5 * q[h] @ K[0, 0] + np.log(n), atol=1e-12)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(2)
    d, n = 16, 40
    K = _rand(rng, 1, n, d)
    V = _rand(rng, 1, n, d)
    q = 200.0 * K[0, 17][None] / np.linalg.norm(K[0, 17])
    K[0] /= np.linalg.norm(K[0], axis=1, keepdims=True)
    o, _ = A.decode(q, K, V, 1.0)
    assert np.allclose(o[0], V[0, 17], atol=1e-6)


def test_gqa_head_map_is_contiguous():
    Hq, Hkv, n, d = 8, 2, 5, 4
    rng = np.random.default_rng(3)
    K = _rand(rng, Hkv, n, d)
    V = np.stack([np.full((n, d), g + 1.0) for g in range(Hkv)])
    o, _ = A.decode(_rand(rng, Hq, d), K, V, 1.0)
    assert np.allclose(o[:, 0], [1, 1, 1, 1, 2, 2, 2, 2])


def _sdpa(q, K, V, scale, mask=None):
    """torch reference: q [Hq, r, d], K/V [Hkv, n, d] -> [Hq, r, d] (float64)."""
    grp = q.shape[0] // K.shape[0]
    Kt = torch.from_numpy(np.repeat(K, grp, axis=0))
    Vt = torch.from_numpy(np.repeat(V, grp, axis=0))
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), Kt, Vt, attn_mask=m, scale=scale).numpy()


def test_decode_matches_torch_sdpa():
    rng = np.random.default_rng(4)
    Hq, Hkv, n, d, t = 8, 2, 300, 32, 5
    q, K, V = _rand(rng, Hq, d), _rand(rng, Hkv, n, d), _rand(rng, Hkv, n, d)
    Kt, Vt = _rand(rng, Hkv, t, d), _rand(rng, Hkv, t, d)
    o, _ = A.decode(q, K, V, 0.17, Kt, Vt)
    ref = _sdpa(q[:, None], np.concatenate([K, Kt], 1), np.concatenate([V, Vt], 1), 0.17)[:, 0]
    assert np.max(np.abs(o - ref)) < 1e-12


def test_verify_matches_torch_sdpa_with_causal_window_mask():
    rng = np.random.default_rng(5)
    Hq, Hkv, N, k, d = 4, 1, 64, 7, 16
    q = _rand(rng, Hq, k, d)
    Kc, Vc, Kw, Vw = _rand(rng, Hkv, N, d), _rand(rng, Hkv, N, d), _rand(rng, Hkv, k, d), _rand(rng, Hkv, k, d)
    mask = np.ones((k, N + k), dtype=bool)
    mask[:, N:] = np.tril(np.ones((k, k), dtype=bool))
    ref = _sdpa(q, np.concatenate([Kc, Kw], 1), np.concatenate([Vc, Vw], 1), d ** -0.5, mask)
    o1, l1 = A.verify(q, Kc, Vc, Kw, Vw, d ** -0.5)
    o2, l2 = A.verify_masked(q, Kc, Vc, Kw, Vw, d ** -0.5)
    assert np.max(np.abs(o1 - ref)) < 1e-12
    assert np.max(np.abs(o2 - ref)) < 1e-12
    assert np.max(np.abs(l1 - l2)) < 1e-12


def test_verify_is_causal_in_the_window():
    rng = np.random.default_rng(6)
    Hq, Hkv, N, k, d = 2, 1, 10, 6, 8
    q = _rand(rng, Hq, k, d)
    Kc, Vc, Kw, Vw = _rand(rng, Hkv, N, d), _rand(rng, Hkv, N, d), _rand(rng, Hkv, k, d), _rand(rng, Hkv, k, d)
    o, _ = A.verify_masked(q, Kc, Vc, Kw, Vw, 0.3)
    i = 2
    Kw2, Vw2 = Kw.copy(), Vw.copy()
    Kw2[:, i + 1:] += 5.0
    Vw2[:, i + 1:] -= 3.0
    o2, _ = A.verify_masked(q, Kc, Vc, Kw2, Vw2, 0.3)
    assert np.array_equal(o[:, : i + 1], o2[:, : i + 1])
    assert not np.allclose(o[:, i + 1:], o2[:, i + 1:])
    Vw3 = Vw.copy()
    Vw3[:, i] += 1.0
    o3, _ = A.verify_masked(q, Kc, Vc, Kw, Vw3, 0.3)
    assert not np.allclose(o[:, i], o3[:, i]) and np.array_equal(o[:, :i], o3[:, :i])


def test_verify_single_row_is_decode():
    rng = np.random.default_rng(7)
    q = _rand(rng, 4, 1, 8)
    Kc, Vc, Kw, Vw = _rand(rng, 2, 9, 8), _rand(rng, 2, 9, 8), _rand(rng, 2, 1, 8), _rand(rng, 2, 1, 8)
    o, lse = A.verify_masked(q, Kc, Vc, Kw, Vw, 0.4)
    od, ld = A.decode(q[:, 0], np.concatenate([Kc, Kw], 1), np.concatenate([Vc, Vw], 1), 0.4)
    assert np.max(np.abs(o[:, 0] - od)) < 1e-14 and np.max(np.abs(lse[:, 0] - ld)) < 1e-13

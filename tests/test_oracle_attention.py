"""Pins of oracle.hadamard and oracle.attention: closed forms, invariants,
and agreement with library routines (scipy's Hadamard, torch's scaled dot
product attention in fp64)."""

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import attention, hadamard


def test_sylvester_closed_forms():
    assert hadamard.sylvester(2).tolist() == [[1, 1], [1, -1]]
    H = hadamard.sylvester(128)
    assert np.array_equal(H @ H.T, 128 * np.eye(128, dtype=np.int64))
    assert np.array_equal(H, scipy.linalg.hadamard(128))
    assert np.array_equal(H, H.T)


def test_transform_involution_and_dense():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((10, 128))
    y = hadamard.transform(x)
    assert np.allclose(hadamard.transform(y), 128 * x, rtol=0, atol=1e-11)
    assert np.allclose(y, x @ scipy.linalg.hadamard(128).T, rtol=0, atol=1e-12)
    # Parseval: ||H x||^2 = 128 ||x||^2
    assert np.allclose((y ** 2).sum(-1), 128 * (x ** 2).sum(-1))


def _rand(rng, T=40, Hkv=2, G=3, D=16):
    q = rng.standard_normal((Hkv * G, D))
    K = rng.standard_normal((T, Hkv, D))
    V = rng.standard_normal((T, Hkv, D))
    return q, K, V


def test_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    q, K, V = _rand(rng, T=1)
    out = attention.attend(q, K, V, 0.3)
    G = q.shape[0] // K.shape[1]
    for h in range(q.shape[0]):
        assert np.allclose(out[h], V[0, h // G])


def test_uniform_scores_give_mean():
    rng = np.random.default_rng(2)
    q, K, V = _rand(rng)
    K[:] = K[0]
    out = attention.attend(q, K, V, 0.7)
    G = q.shape[0] // K.shape[1]
    for h in range(q.shape[0]):
        assert np.allclose(out[h], V[:, h // G].mean(0))
    out0 = attention.attend(np.zeros_like(q), rng.standard_normal(K.shape), V, 1.0)
    for h in range(q.shape[0]):
        assert np.allclose(out0[h], V[:, h // G].mean(0))


def test_two_token_closed_form():
    q = np.array([[1.0, 2.0]])
    K = np.array([[[0.5, 0.0]], [[0.0, -1.0]]])
    V = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    s1, s2 = 0.5 * 0.5, 0.5 * -2.0
    p1 = 1.0 / (1.0 + np.exp(s2 - s1))
    out = attention.attend(q, K, V, 0.5)
    assert np.allclose(out[0], [p1, 1 - p1], rtol=0, atol=1e-15)


def test_shift_and_permutation_invariance():
    rng = np.random.default_rng(3)
    q, K, V = _rand(rng)
    base = attention.attend(q, K, V, 0.25)
    a = rng.standard_normal(K.shape[2])
    assert np.allclose(attention.attend(q, K + a, V, 0.25), base)
    perm = rng.permutation(K.shape[0])
    assert np.allclose(attention.attend(q, K[perm], V[perm], 0.25), base)


def test_gqa_equals_repeated_kv():
    rng = np.random.default_rng(4)
    q, K, V = _rand(rng, Hkv=3, G=4)
    out = attention.attend(q, K, V, 0.2)
    rep = attention.attend(q, np.repeat(K, 4, axis=1), np.repeat(V, 4, axis=1), 0.2)
    assert np.allclose(out, rep)


def test_matches_torch_sdpa():
    rng = np.random.default_rng(5)
    q, K, V = _rand(rng, T=77, Hkv=2, G=4, D=128)
    sm = 1 / np.sqrt(128)
    out = attention.attend(q, K, V, sm)
    G = 4
    tq = torch.from_numpy(q)[:, None, :]                       # [Hq, 1, D]
    tK = torch.from_numpy(np.repeat(K, G, axis=1)).permute(1, 0, 2).contiguous()
    tV = torch.from_numpy(np.repeat(V, G, axis=1)).permute(1, 0, 2).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tK, tV, scale=sm)[:, 0, :]
    assert np.allclose(out, ref.numpy(), rtol=0, atol=1e-12)


def test_empty_cache_rejected():
    with pytest.raises(ValueError):
        attention.attend(np.zeros((1, 4)), np.zeros((0, 1, 4)), np.zeros((0, 1, 4)), 1.0)

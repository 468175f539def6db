"""Pins of oracle.kvarn and oracle.cobra: orthogonality closed forms, the
rotated/rank-space attention identities, and the exact-attention special
cases."""

import numpy as np
import scipy.linalg

from oracle import attention, cobra, hadamard, kvarn
from oracle.codecs import encode_rows, decode_rows
from oracle.rounding import rn16


def _w(rng):
    return (1.0 / np.exp(rng.normal(0, 1, 128))).astype(np.float32)


def test_kvarn_roundtrip_and_attention_identity():
    rng = np.random.default_rng(0)
    w = _w(rng)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    y = kvarn.rotate(x, w)
    assert np.allclose(kvarn.unrotate(y, w), x, rtol=0, atol=1e-12)
    # <q, x> = <H (q / w) / 128, y>: the rotated-space score identity
    q = rng.standard_normal(128)
    qp = hadamard.transform(q / w.astype(np.float64)) / 128
    assert np.allclose(y @ qp, x.astype(np.float64) @ q, rtol=1e-12, atol=1e-12)
    # the rotation spreads an outlier channel over every channel
    xo = np.zeros(128)
    xo[7] = 30.0
    assert np.allclose(np.abs(kvarn.rotate(xo, np.ones(128))), 30.0)


def test_kvarn_f16_codec_attention_equals_plain():
    # F16 storage in the rotated basis: attention over the reconstruction equals
    # attention over the inputs up to binary16 rounding of the rotated values
    rng = np.random.default_rng(1)
    w = _w(rng)
    x = rng.standard_normal((64, 1, 128)).astype(np.float32)
    v = rng.standard_normal((64, 1, 128)).astype(np.float32)
    q = rng.standard_normal((2, 128))
    y = kvarn.rotate(x[:, 0], w)
    xt = kvarn.unrotate(rn16(y).astype(np.float64), w)[:, None, :]
    exact = attention.attend(q, x, v, 1 / np.sqrt(128))
    approx = attention.attend(q, xt, v, 1 / np.sqrt(128))
    assert np.max(np.abs(exact - approx)) < 2e-3
    xt64 = kvarn.unrotate(y, w)[:, None, :]
    assert np.allclose(attention.attend(q, xt64, v, 1 / np.sqrt(128)), exact, atol=1e-12)


def _basis(rng):
    Z = rng.standard_normal((128, 128))
    Q, R = np.linalg.qr(Z)
    return Q * np.sign(np.diag(R))


def test_cobra_projection_properties():
    rng = np.random.default_rng(2)
    U = _basis(rng)
    for r in (16, 32, 64, 128):
        P = cobra.projection(U, r).astype(np.float64)
        assert P.shape == (128, r)
        # columns orthonormal up to binary16 rounding of the entries
        assert np.max(np.abs(P.T @ P - np.eye(r))) < 4e-3
        # same span as the kept directions of U (Hadamard mixes within the span)
        Pk = U[:, :r] @ scipy.linalg.hadamard(r) / np.sqrt(r)
        assert np.allclose(P, Pk, rtol=0, atol=2 ** -11 * np.max(np.abs(Pk)) + 1e-12)
        assert np.array_equal(P, rn16(Pk).astype(np.float64))


def test_cobra_full_rank_fp64_is_exact_and_low_rank_closed_form():
    rng = np.random.default_rng(3)
    U = _basis(rng)
    x = rng.standard_normal((30, 1, 128))
    v = rng.standard_normal((30, 1, 128))
    q = rng.standard_normal((3, 128))
    H = hadamard.sylvester(128) / np.sqrt(128)
    P = U @ H                                        # fp64, r = 128: orthogonal
    xr = cobra.reconstruct(cobra.project(x, P), P)
    assert np.allclose(xr, x, atol=1e-12)
    r = 32
    Pr = U[:, :r] @ (hadamard.sylvester(r) / np.sqrt(r))
    kr = cobra.reconstruct(cobra.project(x, Pr), Pr)
    assert np.allclose(kr, x @ (U[:, :r] @ U[:, :r].T), atol=1e-12)   # K P P^T
    a = attention.attend(q, kr, cobra.reconstruct(cobra.project(v, Pr), Pr), 0.1)
    b = attention.attend(q, x @ Pr @ Pr.T, v @ Pr @ Pr.T, 0.1)
    assert np.allclose(a, b, atol=1e-12)
    # rank-space score identity <P^T q, u> = <q, P u>
    u = cobra.project(x[:, 0], Pr)
    assert np.allclose(u @ (Pr.T @ q[0]), cobra.reconstruct(u, Pr) @ q[0])


def test_cobra_block_coding_of_coordinates():
    rng = np.random.default_rng(4)
    U = _basis(rng)
    P = cobra.projection(U, 16)
    u = cobra.project(rng.standard_normal((8, 128)), P)
    enc = encode_rows(u, "q4_1", block_len=cobra.block_len(16))
    assert enc["codes"].shape == (8, 16) and enc["scales"].shape == (8, 1)
    back = decode_rows(enc, "q4_1", block_len=16, rounded=False)
    d = enc["scales"].astype(np.float64)
    assert np.all(np.abs(back - u) <= d / 2 + np.abs(u.min(-1, keepdims=True)
                                                       - enc["mins"].astype(np.float64)) + 1e-6)


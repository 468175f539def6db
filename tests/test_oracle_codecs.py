"""Pins of oracle.codecs: brute force over exact rationals, error bounds,
idempotence, degenerate blocks, hand-worked blocks, and the binary32
exactness preconditions a device encoder relies on."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import codecs
from oracle.codecs import decode_0, decode_1, encode_0, encode_1, encode_rows, decode_rows
from tests.exact import rn16_exact, rn32_exact

B0 = [8, 6, 5, 4, 3, 2]
B1 = [8, 6, 5, 4, 3, 2, 1]


def _block(rng, L=32, heavy=True):
    x = rng.standard_t(4, L) if heavy else rng.standard_normal(L)
    x = x * np.exp(rng.normal(0, 1))
    return x.astype(np.float32).astype(np.float64)


def _argmin_code(x, d, lo, hi):
    """Code in [lo, hi] nearest x/d, exact; ties to the even code."""
    best = None
    for c in range(lo, hi + 1):
        err = abs(Fraction(x) - c * d)
        key = (err, c % 2)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


@pytest.mark.parametrize("b", B0)
def test_encode_0_brute_force(b):
    rng = np.random.default_rng(10 + b)
    qm = 2 ** (b - 1) - 1
    for trial in range(6):
        x = _block(rng, 32)
        if trial == 5:  # plant exact ties: x = (k + 1/2) d with d forced to d0
            d0 = float(np.float16(0.37))
            x = np.zeros(32)
            x[:8] = (np.arange(8) % qm + 0.5 - qm // 2) * d0
            x[8] = qm * d0
        d, q = encode_0(x[None, :], b)
        amax = max(abs(Fraction(float(v))) for v in x)
        d_exact = rn16_exact(amax / qm)
        assert Fraction(float(d[0])) == d_exact
        for i, v in enumerate(x):
            want = 0 if d_exact == 0 else _argmin_code(float(v), d_exact, -qm, qm)
            assert q[0, i] == want, (b, i, v, q[0, i], want)


@pytest.mark.parametrize("b", B1)
def test_encode_1_brute_force(b):
    rng = np.random.default_rng(20 + b)
    L = 2 ** b - 1
    for trial in range(6):
        x = _block(rng, 32, heavy=(trial % 2 == 0))
        d, m, u = encode_1(x[None, :], b)
        fx = [Fraction(float(v)) for v in x]
        m_exact = rn16_exact(min(fx))
        assert Fraction(float(m[0])) == m_exact
        y = [rn32_exact(v - m_exact) for v in fx]
        R = rn32_exact(max(fx) - m_exact)
        d_exact = rn16_exact(R / L)
        assert Fraction(float(d[0])) == d_exact
        for i in range(32):
            want = 0 if d_exact == 0 else _argmin_code(y[i], d_exact, 0, L)
            assert u[0, i] == want


@pytest.mark.parametrize("b", B0)
def test_encode_0_error_bound_and_no_clamp(b):
    rng = np.random.default_rng(30 + b)
    x = rng.standard_t(4, (4000, 32)) * np.exp(rng.normal(0, 2, (4000, 1)))
    x = x.astype(np.float32).astype(np.float64)
    d, q = encode_0(x, b)
    dd = d.astype(np.float64)
    normal = dd >= 2.0 ** -14
    err = np.abs(x - decode_0(d, q))
    assert np.all(err[normal] <= dd[normal, None] / 2)
    qm = 2 ** (b - 1) - 1
    unclamped = np.rint(x[normal] / dd[normal, None])
    assert np.all(np.abs(unclamped) <= qm)


@pytest.mark.parametrize("b", B1)
def test_encode_1_error_bound(b):
    rng = np.random.default_rng(40 + b)
    x = rng.standard_t(4, (4000, 32)) * np.exp(rng.normal(0, 2, (4000, 1)))
    x = x.astype(np.float32).astype(np.float64)
    d, m, u = encode_1(x, b)
    dd = d.astype(np.float64)
    xr = decode_1(d, m, u, rounded=True)
    bound = (dd[:, None] / 2 + np.abs(x.min(-1) - m.astype(np.float64))[:, None]
             + np.spacing(np.abs(xr).astype(np.float32)).astype(np.float64)
             + np.spacing(np.abs(x).astype(np.float32)).astype(np.float64))
    normal = dd >= 2.0 ** -14
    assert np.all(np.abs(x - xr)[normal] <= bound[normal])


@pytest.mark.parametrize("codec", [c for c in codecs.CODECS if c != "f16"])
def test_idempotent(codec):
    rng = np.random.default_rng(50)
    x = (rng.standard_normal((500, 128)) * 3).astype(np.float32).astype(np.float64)
    e1 = encode_rows(x, codec)
    xr = decode_rows(e1, codec, rounded=True)
    e2 = encode_rows(xr, codec)
    assert np.array_equal(e1["codes"], e2["codes"])
    assert np.array_equal(e1["scales"], e2["scales"])


def test_degenerate_blocks():
    z = np.zeros((1, 32))
    d, q = encode_0(z, 4)
    assert d[0] == 0 and not q.any()
    c = np.full((1, 32), 1.25)
    d, m, u = encode_1(c, 3)
    assert d[0] == 0 and m[0] == np.float16(1.25) and not u.any()
    assert np.all(decode_1(d, m, u) == 1.25)


def test_hand_worked_q4_0_block():
    # amax 7 -> d = 7/7 = 1; codes are the nearest integers, ties to even.
    x = np.array([[0.5, 1.5, 2.5, -0.5, -1.5, 7.0, -7.0, 3.49] + [0.0] * 24])
    d, q = encode_0(x, 4)
    assert d[0] == 1.0
    assert list(q[0, :8]) == [0, 2, 2, 0, -2, 7, -7, 3]


def test_hand_worked_q2_0_is_ternary():
    # qmax = 1: d = amax, codes in {-1, 0, 1}; |x| = d/2 is a tie -> 0 (even)
    x = np.array([[2.0, -2.0, 1.0, -1.0, 1.01, 0.99] + [0.0] * 26])
    d, q = encode_0(x, 2)
    assert d[0] == 2.0
    assert list(q[0, :6]) == [1, -1, 0, 0, 1, 0]


def test_hand_worked_q2_1_block():
    # min 1, max 4 -> m = 1, R = 3, d = 3/3 = 1, u = x - 1
    x = np.array([[1.0, 2.0, 3.0, 4.0, 2.5, 3.5] + [1.0] * 26])
    d, m, u = encode_1(x, 2)
    assert (d[0], m[0]) == (1.0, 1.0)
    assert list(u[0, :6]) == [0, 1, 2, 3, 2, 2]   # 1.5 -> 2 (even), 2.5 -> 2 (even)


def test_signed_max_variant_is_rejected_by_bound():
    # the levels -2^(b-1)..2^(b-1)-1 with d = amax / 2^(b-1) break |x - x^| <= d/2
    x = np.array([[-8.0, 7.9] + [0.0] * 30])
    d, q = encode_0(x, 4)
    assert np.all(np.abs(x - decode_0(d, q)) <= d.astype(np.float64)[:, None] / 2)


def test_binary32_division_reaches_exact_codes():
    # rne(fl32(x / d)) == rne(x / d) and RN16(fl32(a / qmax)) == RN16(a / qmax)
    rng = np.random.default_rng(60)
    x = (rng.standard_t(4, 200000) * np.exp(rng.normal(0, 1.5, 200000)))
    x = np.clip(x, -60000, 60000).astype(np.float32)
    for qm in (1, 3, 7, 15, 31, 127, 255):
        d = np.abs(x[: len(x) // 32 * 32].reshape(-1, 32)).max(-1).astype(np.float64) / qm
        d16 = d.astype(np.float16)
        d16 = np.where(d16 == 0, np.float16(1.0), d16)
        d32 = (np.abs(x[: len(x) // 32 * 32].reshape(-1, 32)).max(-1) / np.float32(qm))
        assert np.array_equal(d32.astype(np.float16), d.astype(np.float16))
        xs = x[: len(x) // 32 * 32].reshape(-1, 32)
        q32 = np.rint(xs / d16.astype(np.float32)[:, None])
        q64 = np.rint(xs.astype(np.float64) / d16.astype(np.float64)[:, None])
        assert np.array_equal(q32, q64)
    # planted exact ties survive binary32 division
    d = np.float32(np.float16(0.3))
    t = ((np.arange(-20, 20) + 0.5) * np.float64(d)).astype(np.float32)
    assert np.array_equal(np.rint(t / d), np.rint(t.astype(np.float64) / np.float64(d)))

"""Pins of oracle.rounding against exact rational rounding."""

from fractions import Fraction

import numpy as np
import pytest

import torch

from oracle.rounding import bf16_bits, f16_bits, f16_from_bits, rbf16, rn16, rn32, rne
from tests.exact import rbf16_exact, rn16_exact, rn32_exact, rne_int


def _samples(rng, n):
    # mix of magnitudes, fp16 midpoints +- tiny offsets, subnormal range
    a = rng.standard_normal(n) * np.exp(rng.uniform(-20, 12, n))
    h = rng.standard_normal(n).astype(np.float16).astype(np.float64)
    ulp = np.spacing(np.abs(h).astype(np.float16)).astype(np.float64)
    mids = h + ulp / 2
    near = mids + rng.choice([-1, 1], n) * np.abs(mids) * 2.0 ** -45
    return np.concatenate([a, mids, near, [0.0, -0.0, 65504.0, 65519.99, 6.0e-8, 3.0e-8]])


@pytest.mark.filterwarnings("ignore:overflow")
def test_rn16_matches_exact_rational():
    rng = np.random.default_rng(1)
    xs = _samples(rng, 400)
    got = rn16(xs)
    for x, g in zip(xs, got):
        want = rn16_exact(Fraction(float(x)))
        if isinstance(want, float):
            assert np.isinf(g) and np.sign(g) == np.sign(want)
        else:
            assert Fraction(float(g)) == want, (x, g, want)


def test_rn32_matches_exact_rational():
    rng = np.random.default_rng(2)
    xs = rng.standard_normal(400) * np.exp(rng.uniform(-30, 30, 400))
    got = rn32(xs)
    for x, g in zip(xs, got):
        assert Fraction(float(g)) == rn32_exact(Fraction(float(x)))


def test_rne_ties_to_even():
    vals = np.array([-2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 3.5, 2.4999, 2.5001])
    assert list(rne(vals)) == [-2, -2, -0, 0, 2, 2, 4, 2, 3]
    for v in vals:
        assert rne(v) == rne_int(Fraction(float(v)))


def test_f16_bits_roundtrip():
    x = np.array([0.0, 1.0, -2.0, 65504.0, 6.1035e-05], dtype=np.float16)
    assert list(f16_bits(x)) == [0x0000, 0x3C00, 0xC000, 0x7BFF, 0x0400]
    assert np.array_equal(f16_from_bits(f16_bits(x)), x)


def test_rbf16_matches_exact_rational_and_torch():
    """bfloat16 rounding (precision-tail format): exact rational rounding of
    binary32 inputs, ties at 2^-8 spacing, subnormals; and torch's own
    float32 -> bfloat16 conversion (round to nearest even) on many values."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(300) * np.exp(rng.uniform(-60, 60, 300))).astype(np.float32)
    ties = np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3 * 2 ** -134, 2 ** -133,
                       (1 + 2 ** -8) * 2 ** -100])
    xs = np.concatenate([x, ties]).astype(np.float64)
    got = rbf16(xs)
    for v, g in zip(xs, got):
        assert Fraction(float(g)) == rbf16_exact(Fraction(float(v))), (v, g)
    assert list(got[-6:-3]) == [1.0, 1 + 2 ** -6, -1.0]
    many = (rng.standard_normal(100000) * np.exp(rng.uniform(-80, 80, 100000))).astype(np.float32)
    ref = torch.from_numpy(many).to(torch.bfloat16)
    assert np.array_equal(bf16_bits(rbf16(many.astype(np.float64))), ref.view(torch.int16).numpy().view(np.uint16))

"""Pins for the L2-norm oracle (oracle/l2norm.py), each against a reference
that does not reuse the oracle's code: exact rational arithmetic (Fraction),
closed forms, and float64 torch on values whose sum of squares is exact.

The pages (RL-Kernel page "H100 canonical CP backward validation", Change and
Timing sections) print no numerical example of the norm, so no pin is a
printed value.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import datagen
from oracle import l2norm as L

RNG = np.random.default_rng(777)


def wide_values(n, rng):
    """float32 values over a wide exponent range, both signs, some zeros."""
    mant = rng.uniform(1.0, 2.0, n)
    exp = rng.integers(-80, 64, n)
    v = (mant * np.exp2(exp) * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    v[rng.random(n) < 0.05] = 0.0
    return v


def exact_square_f32(x: float) -> float:
    # the product of two float32 values has at most 48 significant bits: exact
    # in float64, so one float32 rounding of it is the correctly rounded square
    with np.errstate(over="ignore"):
        return float(np.float32(float(Fraction(float(x)) ** 2)))


def test_squares_are_correctly_rounded():
    v = np.concatenate([wide_values(3000, RNG), np.array([3.0, 2.0 ** -75, 2.0 ** -74, 1.8446743e19, 2.0 ** 64],
                                                         dtype=np.float32)])
    s = L.squares(v)
    for x, got in zip(v.tolist(), s.tolist()):
        assert got == exact_square_f32(x), x


def test_bins_closed_forms():
    b, nn, ni = L.bins([np.array([1.0], np.float32)])
    assert b[127] == 1 << 23 and sum(b) == 1 << 23 and nn == ni == 0
    b, _, _ = L.bins([np.array([3.0, -3.0], np.float32)])       # 9 = 1.125 * 2^3
    assert b[130] == 2 * 0x900000 and sum(b) == 2 * 0x900000
    b, _, _ = L.bins([np.array([2.0 ** -70], np.float32)])      # 2^-140 = 512 * 2^-149 (subnormal)
    assert b[0] == 512 and sum(b) == 512
    assert L.sumsq_from_bins(b, 0, 0) == 2.0 ** -140
    b, _, _ = L.bins([np.array([2.0 ** -70, 3 * 2.0 ** -72, 2.0 ** -63], np.float32)])  # subnormal + normal squares
    assert L.sumsq_from_bins(b, 0, 0) == 2.0 ** -140 + 9 * 2.0 ** -144 + 2.0 ** -126
    b, _, _ = L.bins([np.array([2.0 ** -75], np.float32)])      # 2^-150 rounds to 0 (ties to even)
    assert sum(b) == 0
    b, nn, ni = L.bins([np.array([np.nan, np.inf, -np.inf, 2.0 ** 64, 1.0], np.float32)])
    assert nn == 1 and ni == 3 and b[127] == 1 << 23


def test_sumsq_equals_exact_rational_sum():
    for trial in range(20):
        n = int(RNG.integers(1, 400))
        v = wide_values(n, RNG)
        exact = sum((Fraction(exact_square_f32(x)) for x in v.tolist()), Fraction(0))
        want = float(exact)  # Fraction -> float is correctly rounded
        assert L.sumsq([v]) == want
        assert L.sumsq_from_bins(*L.bins([v])) == want


def test_norm_closed_forms():
    assert L.norm([np.ones(1_000_000, np.float32)]) == (1e6, 1000.0)
    assert L.norm([np.array([3.0, 4.0], np.float32)]) == (25.0, 5.0)
    assert L.norm([np.zeros(10, np.float32)]) == (0.0, 0.0)
    assert L.norm([np.array([], np.float32)]) == (0.0, 0.0)
    v = datagen.grad_values(3, 5000)
    s, n = L.norm([v])
    for k in (-20, -3, 5, 30):
        s2, n2 = L.norm([(v * np.float32(2.0 ** k)).astype(np.float32)])
        assert s2 == s * 4.0 ** k and n2 == n * 2.0 ** k


def test_special_values():
    assert math.isnan(L.norm([np.array([1.0, np.nan], np.float32)])[1])
    assert math.isnan(L.norm([np.array([np.inf, np.nan], np.float32)])[0])
    assert L.norm([np.array([1.0, -np.inf], np.float32)]) == (math.inf, math.inf)
    assert L.norm([np.array([2.0 ** 64], np.float32)])[0] == math.inf          # square overflows float32
    big = np.nextafter(np.float32(2.0 ** 64), np.float32(0))                  # largest float32 below 2^64
    assert L.norm([np.array([big], np.float32)])[0] == exact_square_f32(float(big)) == 2.0 ** 128 - 2.0 ** 105
    assert L.norm([np.array([2.0 ** -75] * 3, np.float32)]) == (0.0, 0.0)     # squares round to 0


def test_several_tensors_equal_their_concatenation_in_any_order():
    parts = [wide_values(int(RNG.integers(0, 300)), RNG) for _ in range(7)]
    whole = np.concatenate(parts)
    want = L.norm([whole])
    assert L.norm(parts) == want
    assert L.norm(parts[::-1]) == want
    assert L.norm([RNG.permutation(whole)]) == want
    b = L.bins(parts)
    assert L.sumsq_from_bins(*b) == want[0]


def test_against_torch_float64_on_exactly_summable_values():
    import torch
    # BF16-derived values with exponents in a 40-bit window: every partial sum of
    # the squares is exact in float64, so torch's float64 sum is exact too
    v = datagen.grad_values(11, 200_000, sigma=1.0)
    v = np.clip(v, -64, 64)
    v[np.abs(v) < 2.0 ** -6] = 0.0
    t = torch.from_numpy(v).double()
    want = float((t * t).sum())
    assert L.sumsq([v]) == want
    assert L.norm([v])[1] == float(np.float32(math.sqrt(want)))


def test_microbench_values_are_bf16_derived():
    v = datagen.grad_values(7, 1 << 16)
    assert np.array_equal(datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(v)), v)
    s = L.squares(v)
    # squares of BF16 values are exact in float32
    assert all(float(a) == float(x) * float(x) for a, x in zip(s[:2000].tolist(), v[:2000].tolist()))


def test_final_square_root_is_rounded_twice_from_float64():
    """norm = fl32(sqrt(fl64(S))): checked with 60-digit square roots rounded
    to float64 and then to float32."""
    import mpmath
    rng = np.random.default_rng(5)
    vals = np.ldexp(rng.uniform(1.0, 2.0, 3000), rng.integers(-200, 200, 3000))
    with mpmath.workdps(60):
        for s in vals.tolist():
            r64 = float(mpmath.sqrt(mpmath.mpf(s)))  # mpf -> float rounds to nearest
            assert L.norm_from_sumsq(s) == float(np.float32(r64)), s
    assert L.norm_from_sumsq(math.inf) == math.inf and math.isnan(L.norm_from_sumsq(math.nan))

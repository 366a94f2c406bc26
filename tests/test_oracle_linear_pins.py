"""Pins for the LM-head linear oracle (oracle/linear.py), against references that
do not reuse its code: exact rational dot products (Fraction), exact rational
round-to-nearest-even into 8 significant bits, and the logprob oracle's own
pins for the last step.

The pages (RL-Kernel page "Reproduce and profile the Qwen3-8B TP4/CP2
experiment", section "Capture logs, status, and validation evidence") name the
`linear-logp` backend but print no numerical example, so no pin is a printed
value.
"""
import math
from fractions import Fraction

import numpy as np

import datagen
from oracle import linear as LIN
from oracle import logp as O


def frac_bf16(bits):
    return Fraction(float(datagen.bf16_bits_to_f32(np.array([bits], np.uint16))[0]))


def rne8(q: Fraction) -> Fraction:
    """Round a positive rational to 8 significant bits, ties to even."""
    e = 0
    while q >= 256:
        q /= 2
        e += 1
    while q < 128:
        q *= 2
        e -= 1
    fl = math.floor(q)
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return Fraction(fl) * Fraction(2) ** e


def test_dot_products_are_exact_sums():
    rng = np.random.default_rng(9)
    h = datagen.f32_to_bf16_bits(rng.normal(0, 1, (3, 64)).astype(np.float32))
    w = datagen.f32_to_bf16_bits(rng.normal(0, 0.1, (5, 64)).astype(np.float32))
    acc = LIN.acc_exact(h, w)
    for i in range(3):
        for j in range(5):
            exact = sum(frac_bf16(h[i, k]) * frac_bf16(w[j, k]) for k in range(64))
            assert abs(Fraction(acc[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_bf16_rounding_is_nearest_even_on_8_significant_bits():
    rng = np.random.default_rng(4)
    vals = np.concatenate([rng.normal(0, 3, 4000), rng.normal(0, 1e-30, 200), rng.normal(0, 1e30, 200),
                           # exact ties: 8-bit significands plus half a unit in the last place
                           (np.arange(128, 256) + 0.5) * 2.0 ** -7, -(np.arange(128, 256) + 0.5) * 2.0 ** 3])
    bits = LIN.round_bf16(vals)
    for v, b in zip(vals.tolist(), bits.tolist()):
        want = rne8(Fraction(abs(v)))
        want = want if v >= 0 else -want
        assert frac_bf16(b) == want, (v, hex(b))


def test_bf16_rounding_special_values():
    bits = LIN.round_bf16(np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.4e38, -3.4e38, 1e-45, 2.0 ** -134,
                                    3 * 2.0 ** -134]))
    assert list(bits[:4]) == [0x0000, 0x8000, 0x7F80, 0xFF80] and bits[4] == 0x7FC0
    assert bits[5] == 0x7F80 and bits[6] == 0xFF80       # beyond the largest BF16 (3.3895e38) after rounding
    assert bits[7] == 0x0000 and bits[8] == 0x0000        # below half of the smallest subnormal 2^-133, and a tie to 0
    assert bits[9] == 0x0002                              # 1.5 * 2^-133 rounds to 2 * 2^-133


def test_exact_inputs_give_exact_bf16_logits():
    h, w = datagen.linear_exact_inputs(3, 20, 448, 300)
    acc = LIN.acc_exact(h, w)
    assert np.all(acc == np.round(acc * 16) / 16) and np.abs(acc).max() <= 3 * 80 / 16
    x = LIN.logits_bf16(h, w, 320)
    assert np.array_equal(datagen.bf16_bits_to_f32(x[:, :300]).astype(np.float64), acc)
    assert np.all(x[:, 300:] == 0xFF80)


def test_linear_logp_is_the_logprob_of_the_rounded_logits():
    """Composition: the target's logit is the exact dot product rounded once to
    8 significant bits (exact rationals), and the logprob is the logprob
    oracle's value on those logits (pinned in test_oracle_pins.py)."""
    h, w = datagen.linear_inputs(5, 6, 256, 1000)
    t = np.array([1.0, 0.7, 1.3, 0.0, 0.7, 2.0], np.float32)
    tg = np.array([0, 999, 500, 3, 7, 123], np.int64)
    got, _ = LIN.linear_logp(h, w, 1024, t, tg)
    lg = LIN.logits_bf16(h, w, 1024)
    for i in range(6):
        for j in (int(tg[i]), 0, 1, 998):
            e = sum(frac_bf16(h[i, k]) * frac_bf16(w[j, k]) for k in range(256))
            want_x = (rne8(abs(e)) * (1 if e > 0 else -1)) if e != 0 else Fraction(0)
            assert frac_bf16(lg[i, j]) == want_x
        ref, _ = O.ref_logp_row(lg[i], 1000, float(t[i]), int(tg[i]))
        assert got[i] == ref

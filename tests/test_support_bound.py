"""The bracket the nucleus kernel puts around a row's total mass, checked on the host.

The kernel decides the top-p boundary from the thresholds of both ends of a
bracket [Z (1 - eps), Z (1 + eps)] built from the float32 shard sums l_s
(reference exponents r_s), where the exact total is the integer
Z = sum floor(2^(fl32(x c - R)) 2^40) over the row's tokens (R from the row
maximum). The decision is exact only if the bracket holds Z. This test rebuilds
both numbers the way the kernel computes them: the shard sums in its frozen
order (lane l owns vectors l, l+64, ...; eight accumulators per lane fed in
vector order; lane total ((a0+a1)+(a2+a3))+((a4+a5)+(a6+a7)); the 64 lanes
folded by halving), float32 exp2 standing in for v_exp_f32 (both within a few
ulp). It then checks the gap is far inside the bound the kernel uses.
Rows are the benchmark's shapes and distributions (152576 columns in 8 shards
of 19072, 151936 real; N(0, 2.5^2) BF16 logits, with and without a +8 spike;
T 0.7, 1.0, 1.3) plus a row whose shards peak long after their first chunk,
so r_s sits far below R.
"""
import math

import numpy as np
import pytest

import datagen

VOCAB_REAL = 151936
SHARD = 19072
WAVE = 64


def f32(x):
    return np.float32(x)


def fl32_fma(x, c, r):
    # x is a BF16 value and c a float32: the product is exact in float64, and
    # x*c - r is rounded once more to float32
    return (x.astype(np.float64) * np.float64(c) - np.float64(r)).astype(np.float32)


def shard_sum(xs, c, r):
    """Float32 sum of 2^(fl32(x c - r)) over one shard's real columns, in the kernel's order."""
    nvec = len(xs) // 8
    terms = np.exp2(fl32_fma(xs, c, r)).astype(np.float32).reshape(nvec, 8)
    per_lane = -(-nvec // WAVE)
    padded = np.zeros((per_lane * WAVE, 8), dtype=np.float32)  # missing vectors add +0
    padded[:nvec] = terms
    padded = padded.reshape(per_lane, WAVE, 8)
    acc = np.zeros((WAVE, 8), dtype=np.float32)
    for v in range(per_lane):
        acc = (acc + padded[v]).astype(np.float32)
    a = acc
    lane = ((a[:, 0] + a[:, 1]) + (a[:, 2] + a[:, 3])) + ((a[:, 4] + a[:, 5]) + (a[:, 6] + a[:, 7]))
    lane = lane.astype(np.float32)
    while len(lane) > 1:
        h = len(lane) // 2
        lane = (lane[:h] + lane[h:]).astype(np.float32)
    return float(lane[0])


def totals(x, t):
    c = f32(f32(1.4426950408889634) / f32(t))
    zf_terms = []
    for s in range(8):
        xs = x[s * SHARD: min((s + 1) * SHARD, len(x))]
        m0 = float(xs[:2048].max())  # the first group of 4 vectors per lane
        r = math.ceil(float(f32(f32(m0) * c)))
        zf_terms.append((shard_sum(xs, c, r), r))
    R = math.ceil(float(f32(f32(x.max()) * c)))
    w = np.exp2(fl32_fma(x, c, R)).astype(np.float32).astype(np.float64)
    z_int = int(np.floor(w * 2.0 ** 40).astype(np.int64).sum())
    zf = sum(math.ldexp(l, r - R + 40) for l, r in zf_terms)
    dmax = max(R - r for l, r in zf_terms if l > 0)
    return zf, z_int, dmax


def kernel_eps(shard_width, vocab_real, dmax):
    """The kernel's bracket half-width: float-sum depth, half an ulp of the
    largest shard-argument magnitude max(31, D + 1) and of 31 for the weight
    argument, v_exp_f32, the neglected tails and the floor, twice."""
    depth = (shard_width // 8 + WAVE) // WAVE + 1 + 3 + 6
    karg = max(31.0, dmax + 1.0)
    half_ulp = math.ldexp(1.0, math.frexp(karg)[1] - 1 - 24)
    return 2.0 * (depth * 2.0 ** -24 + half_ulp + 2.0 ** -20 + 2.0 ** -22 + 2.0 ** -30 +
                  1.25 * vocab_real * 2.0 ** -39)


def rows():
    out = []
    for i, (t, spike) in enumerate([(0.7, 8.0), (0.7, None), (1.0, None), (1.3, None), (1.3, 8.0)]):
        bits, _, _ = datagen.row_values((777, i), VOCAB_REAL, 2.5, spike)
        out.append((f"sigma 2.5 T {t} spike {spike}", datagen.bf16_bits_to_f32(bits), t))
    # every shard peaks at its end: r_s comes from a first chunk far below the row maximum
    bits, _, _ = datagen.row_values((777, 99), VOCAB_REAL, 2.5, None)
    x = datagen.bf16_bits_to_f32(bits).copy()
    for s in range(8):
        x[min((s + 1) * SHARD, VOCAB_REAL) - 1] = np.float32(20.0 + s)
    out.append(("late shard maxima", x, 0.7))
    return out


@pytest.mark.parametrize("name,x,t", rows(), ids=[r[0] for r in rows()])
def test_shard_sums_bracket_the_integer_total(name, x, t):
    zf, z_int, dmax = totals(x, t)
    rel = abs(zf - z_int) / z_int
    eps = kernel_eps(SHARD, VOCAB_REAL, dmax)
    assert z_int >= 2 ** 39
    # the kernel brackets with eps; the observed gap must sit far inside it
    assert rel < eps / 8, (name, rel, eps)
    assert z_int >= int(zf * (1.0 - eps)) and z_int <= int(zf * (1.0 + eps)) + 1

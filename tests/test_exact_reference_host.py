"""The exact-mass reference of rlk_logp_nucleus, checked on the host.

On a row that needs a support search and whose tokens all lie in the support's
window of BF16 classes, the nucleus entry point takes the reference log-sum-exp
from the same integers as the support: every token weighs
floor(2^(fl32(x*c - R)) * 2^40) with c = fl32(log2(e)/T) and R = ceil(fl32(M*c))
for the row maximum M, the row's total is Z = sum of the weights, and
lse = ln 2 * (R + log2(Z) - 40). This test rebuilds those integers the way the
kernel forms them (the product x*c of a BF16 value and a float32 is exact in
float64, and the argument is rounded once to float32, as the kernel's fused
multiply-add does; float32 exp2 stands in for v_exp_f32, both within a few
ulp) and checks:

- the floor loses less than one 2^-40 unit per token, against the unrounded
  sum of the same float32 weights (an exact property of the truncation);
- Z >= 2^39 (the maximum's own weight is at least one half);
- lse lies within 4e-6 of the oracle's float64 log-sum-exp on the benchmark's
  rows (T 0.7 with the +8 spike; the per-request temperatures 0.7, 1.0 and
  1.3), well inside the 2e-5 tolerance: truncation (under 151936 / 2^39 =
  2.8e-7 relative), the rounding of the exponent argument and of exp2, and the
  float32 rounding of c that the float32 shard sums of rlk_logp_full carry
  too.
"""
import math

import numpy as np
import pytest

import datagen
from oracle import logp as O

LOG2E_F32 = np.float32(1.44269504088896340736)


def exact_lse(x: np.ndarray, t: float):
    """(lse, Z, unrounded sum, R) from the kernel's integer weights of the finite tokens x (float32)."""
    c = np.float32(LOG2E_F32 / np.float32(t))
    m = np.float32(x.max())
    r = float(np.ceil(np.float32(m * c)))
    arg = (x.astype(np.float64) * np.float64(c) - r).astype(np.float32)  # one rounding, as fmaf
    w = np.exp2(arg)  # float32
    scaled = w.astype(np.float64) * 2.0 ** 40  # exact: a power-of-two scaling of a float32
    units = np.floor(scaled)
    z = int(units.astype(np.uint64).sum(dtype=np.uint64))
    lse = (r + (math.log2(z) - 40.0)) * math.log(2.0)
    return lse, z, math.fsum(scaled.tolist()), r


def rows_of(w, idx):
    out = []
    for i in idx:
        bits, _, _ = w.row(i)
        x = datagen.bf16_bits_to_f32(bits[: w.vocab_real])
        out.append((int(i), x, float(w.temperature[i]), bits))
    return out


CASES = [
    ("full T 0.7 + spike", datagen.full(), range(0, 8192, 512)),
    ("per-request", datagen.per_request(), [r * 128 + 7 for r in range(12)]),
]


@pytest.mark.parametrize("name,w,idx", CASES, ids=[c[0] for c in CASES])
def test_exact_mass_reference_matches_the_oracle(name, w, idx):
    worst = 0.0
    for i, x, t, bits in rows_of(w, idx):
        fin = x[np.isfinite(x)]
        lse, z, unrounded, _ = exact_lse(fin, t)
        lost = unrounded - z
        assert -64.0 <= lost < fin.size + 64.0, (name, i, lost)  # fp64 sum of the unrounded weights: +-64 units
        assert z >= 2 ** 39, (name, i, z)
        _, want = O.ref_logp_row(bits, w.vocab_real, t, 0)
        err = abs(lse - want)
        worst = max(worst, err)
        assert err <= 4e-6, (name, i, t, lse, want)
    print(f"{name}: largest |lse_exact - lse_oracle| {worst:.2e}")


def test_truncation_loses_under_one_unit_per_fractional_weight():
    """A row of 151936 tokens spread over about 30 binades of weight below one
    maximal token. A weight of 2^24 units or more is an integer already (its
    float32 has no fraction bits left), so only the smaller ones lose a
    fraction to the floor: the loss is below one unit per such token, and
    about half a unit on average."""
    rng = np.random.default_rng(11)
    x = np.concatenate([[np.float32(8.0)], rng.uniform(-6.0, 8.0, 151935).astype(np.float32)])
    x = datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(x))
    lse, z, unrounded, r = exact_lse(x, 0.7)
    c = np.float32(LOG2E_F32 / np.float32(0.7))
    scaled = np.exp2((x.astype(np.float64) * np.float64(c) - r).astype(np.float32)).astype(np.float64) * 2.0 ** 40
    n_frac = int(np.count_nonzero(scaled < 2.0 ** 24))
    lost = unrounded - z
    assert 0.25 * n_frac < lost < n_frac + 64.0, (lost, n_frac)
    want = float(np.log(np.sum(np.exp(x.astype(np.float64) / np.float64(np.float32(0.7))))))
    assert abs(lse - want) <= 4e-6

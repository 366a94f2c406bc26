"""Pins for the oracle's top-p ambiguity band (``NucleusInfo.ambiguous`` and
``NucleusInfo.alternatives``).

The band is a reading of the pages, not something they define: page
"Configurable H100 consistency runs", sampling paragraph, puts top-p in
(0, 1] and computes the support from the real vocabulary; the mode/KL
paragraph keeps the policy logprob on its actual top-p/top-k support. A GPU
decides the top-p cut on masses that differ from the float64 ones by about
1e-7 relative, so a row whose cumulative fraction at the boundary class lies
within 2e-6 of p may legitimately take the neighbouring cut. The oracle flags
such rows and lists the policy value under each neighbouring cut.

These pins place p at a chosen exact distance from the class edges of small
rows whose cumulative fractions are computed independently (mpmath at 60
digits), and check:
- ``ambiguous`` is set exactly when an edge lies within the band on the side
  that has a neighbouring cut (inside: delta/2; outside: 2*delta);
- each alternative equals the policy value under the support one class
  earlier or later, where that support is found by exhaustive subset
  enumeration (the smallest upper-closed token set whose exact mass reaches a
  p' placed strictly between the neighbouring cumulative fractions) and the
  value by a 60-digit log-sum over it.
"""
import itertools
import math

import mpmath
import numpy as np
import pytest

import datagen
from oracle import logp as O

BAND = 2e-6


def _row(values_with_counts):
    vals = []
    for v, c in values_with_counts:
        vals += [v] * c
    rng = np.random.default_rng(len(vals))
    vals = np.array(vals, dtype=np.float32)[rng.permutation(len(vals))]   # classes not contiguous
    return datagen.f32_to_bf16_bits(vals), vals.astype(np.float64)


# Rows at T = 1 (z = x exactly): distinct values with tie counts, descending.
ROWS = [
    [(2.0, 1), (1.5, 2), (1.0, 3), (0.5, 2), (0.0, 4), (-0.5, 1), (-1.0, 3)],
    [(3.0, 2), (2.75, 1), (1.0, 5), (0.25, 1), (-2.0, 6)],
    [(0.5, 1), (0.0, 1), (-0.25, 1), (-0.5, 1), (-3.0, 2)],
]


def _exact_classes(z, k):
    """Descending distinct values, counts, and the 60-digit cumulative mass
    fractions over the classes that top-k keeps (count reaches k; ties kept)."""
    vals = sorted(set(z), reverse=True)
    counts = [int(np.sum(z == v)) for v in vals]
    r_k = len(vals) - 1
    if k != -1 and k < len(z):
        cum = 0
        for r, c in enumerate(counts):
            cum += c
            if cum >= k:
                r_k = r
                break
    with mpmath.workdps(60):
        m = mpmath.mpf(vals[0])
        w = [c * mpmath.exp(mpmath.mpf(v) - m) for v, c in zip(vals, counts)]
        zk = mpmath.fsum(w[:r_k + 1])
        fr = []
        acc = mpmath.mpf(0)
        for r in range(r_k + 1):
            acc += w[r]
            fr.append(acc / zk)
    return vals, counts, r_k, fr


def _upper_closed(sub, z):
    s = set(sub)
    return all(i in s for j in s for i in range(len(z)) if z[i] >= z[j])


def _enumerated_support(z, allowed, p_exact):
    """Smallest upper-closed subset of ``allowed`` (itself upper-closed) whose
    exact mass reaches ``p_exact`` times the mass of ``allowed``: exhaustive."""
    with mpmath.workdps(60):
        m = mpmath.mpf(max(z))
        mass = {j: mpmath.exp(mpmath.mpf(z[j]) - m) for j in allowed}
        total = mpmath.fsum(mass.values())
        best = None
        for r in range(1, len(allowed) + 1):
            for c in itertools.combinations(sorted(allowed), r):
                if _upper_closed(c, z) and mpmath.fsum(mass[j] for j in c) >= p_exact * total:
                    best = set(c)
                    break
            if best is not None:
                break
    return best


def _policy_on(z, support, t, ref):
    if len(support) == len(z):
        return ref
    if t not in support:
        return float("-inf")
    with mpmath.workdps(60):
        return float(mpmath.mpf(z[t]) - mpmath.log(mpmath.fsum(mpmath.exp(mpmath.mpf(z[j])) for j in support)))


def _cases():
    """(row, top-k, boundary class, side, distance in bands): every class that
    top-k keeps, p placed inside it at delta/2 or 2*delta from its upper edge
    ("before": the fraction before the class) or its lower edge ("at")."""
    out = []
    for ri, spec in enumerate(ROWS):
        n_classes = len(spec)
        for k in (-1, sum(c for _, c in spec[:n_classes - 2]) - 1):
            r_k = _exact_classes(_row(spec)[1], k)[2]
            for b in range(r_k + 1):
                for side, dist in (("before", 0.5), ("before", 2.0), ("at", 0.5), ("at", 2.0)):
                    if side == "before" and b == 0:
                        continue
                    out.append((ri, k, b, side, dist))
    return out


@pytest.mark.parametrize("ri,k,b,side,dist", _cases())
def test_band_flag_and_alternatives(ri, k, b, side, dist):
    bits, z = _row(ROWS[ri])
    V = len(z)
    vals, counts, r_k, fr = _exact_classes(z, k)
    # p at the chosen distance inside the boundary class b, rounded to float32
    with mpmath.workdps(60):
        edge = fr[b - 1] if side == "before" else fr[b]
        want_p = edge + (dist * BAND if side == "before" else -dist * BAND)
        p32 = float(np.float32(float(want_p)))
        pe = mpmath.mpf(p32)
        lo = fr[b - 1] if b > 0 else mpmath.mpf(0)
        assert lo < pe <= fr[b], "p must fall in class b"
        d_before = float(pe - fr[b - 1]) if b > 0 else math.inf    # p minus the fraction before class b
        d_at = float(fr[b] - pe)                                    # the fraction at class b minus p
    if p32 >= 1.0:
        pytest.skip("p rounds to 1 (top-p disabled)")
    flag_before = b > 0 and d_before <= BAND
    flag_at = b < r_k and d_at <= BAND
    # the placements are far from the band's edge, so float rounding cannot matter
    assert abs(d_before - BAND) > 0.2 * BAND and abs(d_at - BAND) > 0.2 * BAND

    x = datagen.bf16_bits_to_f32(bits).astype(np.float64)
    allowed = {j for j in range(V) if x[j] >= vals[r_k]}
    sup_b = {j for j in range(V) if x[j] >= vals[b]}
    # the primary support is also what enumeration gives at this p
    assert _enumerated_support(z, allowed, mpmath.mpf(p32)) == sup_b
    with mpmath.workdps(60):
        sup_earlier = (_enumerated_support(z, allowed, (fr[b - 2] + fr[b - 1]) / 2 if b >= 2 else fr[0] / 2)
                       if b > 0 else None)
        sup_later = _enumerated_support(z, allowed, (fr[b] + fr[b + 1]) / 2) if b < r_k else None
    if sup_earlier is not None:
        assert sup_earlier == {j for j in range(V) if x[j] >= vals[b - 1]}
    if sup_later is not None:
        assert sup_later == {j for j in range(V) if x[j] >= vals[b + 1]}

    order = np.argsort(-x, kind="stable")
    targets = {int(order[0]), int(np.flatnonzero(x == vals[b])[0])}
    if b + 1 < len(vals):
        targets.add(int(np.flatnonzero(x == vals[b + 1])[0]))
    for t in sorted(targets):
        pol, ref, info = O.nucleus_row(bits, V, 1.0, p32, k, t)
        assert info.r_p == b and info.r_star == b
        assert info.ambiguous == (flag_before or flag_at), (d_before, d_at, info.frac_before, info.frac_at)
        want_alts = []
        if flag_before:
            want_alts.append(_policy_on(z, sup_earlier, t, ref))
        if flag_at:
            want_alts.append(_policy_on(z, sup_later, t, ref))
        assert len(info.alternatives) == len(want_alts)
        for got, want in zip(info.alternatives, want_alts):
            if math.isinf(want):
                assert got == want
            else:
                assert abs(got - want) < 1e-12, (got, want)
        assert abs(pol - _policy_on(z, sup_b, t, ref)) < 1e-12 or pol == _policy_on(z, sup_b, t, ref)


def test_band_cases_cover_every_outcome():
    """The placements reach each of: flagged before, flagged at, flagged on
    both sides (none here: classes are wider than the band), not flagged, and a
    flag suppressed at the top-k edge."""
    seen = set()
    for ri, k, b, side, dist in _cases():
        bits, z = _row(ROWS[ri])
        vals, counts, r_k, fr = _exact_classes(z, k)
        with mpmath.workdps(60):
            edge = fr[b - 1] if side == "before" else fr[b]
            p32 = float(np.float32(float(edge + (dist * BAND if side == "before" else -dist * BAND))))
        if p32 >= 1.0:
            continue
        _, _, info = O.nucleus_row(bits, len(z), 1.0, p32, k, 0)
        if info.ambiguous:
            seen.add("flag-" + side)
        elif dist < 1 and side == "at" and b == r_k:
            seen.add("suppressed-at-topk-edge")
        else:
            seen.add("clear")
    assert {"flag-before", "flag-at", "clear", "suppressed-at-topk-edge"} <= seen


def test_band_width_is_a_parameter():
    """A row placed at 3*delta from an edge is flagged under a band of 4*delta
    and not under the default."""
    bits, z = _row(ROWS[0])
    vals, counts, r_k, fr = _exact_classes(z, -1)
    with mpmath.workdps(60):
        p32 = float(np.float32(float(fr[2] + 3 * BAND)))
    _, _, info = O.nucleus_row(bits, len(z), 1.0, p32, -1, 0)
    assert not info.ambiguous
    _, _, info = O.nucleus_row(bits, len(z), 1.0, p32, -1, 0, band=4 * BAND)
    assert info.ambiguous and len(info.alternatives) == 1

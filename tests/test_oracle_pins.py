"""Pins for the CPU oracle: every check here uses a reference that does not
reuse the oracle's code (struct decoding, exact rational rounding, 50-digit
mpmath sums, closed forms, torch's float64 log_softmax, exhaustive subset
enumeration with exact rational masses, the temperature-to-zero limit).

The pages that define the method (RL-Kernel documentation: "Configurable H100
consistency runs", sampling and mode/KL paragraphs; "Reproduce and profile the
Qwen3-8B TP4/CP2 experiment", section "How non-default CUDA topology reuses
TP4/CP2") print no worked numerical example, so no pin here is a printed value.
"""
import itertools
import math
import struct
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import datagen
from oracle import logp as O

RNG = np.random.default_rng(12345)


def bf16(values):
    return datagen.f32_to_bf16_bits(np.asarray(values, dtype=np.float32))


def f32(bits):
    return datagen.bf16_bits_to_f32(bits)


# --------------------------------------------------------------------------- decode

def test_decode_matches_struct_unpack():
    bits = np.concatenate([
        np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4049, 0x7F7F, 0xFF7F, 0x0001, 0x8001,
                  0x0080, 0xFF80, 0x7F80], dtype=np.uint16),
        RNG.integers(0, 0x7F80, size=3000).astype(np.uint16),
        (RNG.integers(0, 0x7F80, size=3000) | 0x8000).astype(np.uint16),
    ])
    got = O.decode_bf16(bits)
    for b, g in zip(bits.tolist(), got.tolist()):
        want = struct.unpack(">f", struct.pack(">HH", b, 0))[0]
        assert (g == want) or (math.isnan(g) and math.isnan(want)), hex(b)
        assert math.copysign(1.0, g) == math.copysign(1.0, want)


# --------------------------------------------------------------------------- fp32 division

def _nearest_f32(q: Fraction) -> float:
    """Round an exact rational to the nearest float32, ties to even (by exhaustive
    comparison of neighbouring float32 values)."""
    c = np.float32(float(q))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    cands = [x for x in cands if np.isfinite(x)]
    best = None
    for x in cands:
        d = abs(Fraction(float(x)) - q)
        key = (d, int(np.array(x, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, x)
    return float(best[1])


@pytest.mark.parametrize("temperature", [0.7, 1.3, 1.0, 0.5, 0.3, 1e-3, 3.0, 0.123456789])
def test_scale_is_correctly_rounded_fp32_division(temperature):
    x = f32(bf16(RNG.normal(0, 4.0, size=400)))
    t32 = np.float32(temperature)
    got = O.scale_fp32(x, temperature)
    for xi, gi in zip(x.tolist(), got.tolist()):
        want = _nearest_f32(Fraction(xi) / Fraction(float(t32)))
        assert gi == want, (xi, temperature)


def test_scale_unit_temperature_is_identity():
    x = f32(bf16(RNG.normal(0, 3.0, size=1000)))
    assert np.array_equal(O.scale_fp32(x, 1.0), x.astype(np.float64))


# --------------------------------------------------------------------------- reference logprob

def _mp_ref(z, t, dps=50):
    with mpmath.workdps(dps):
        s = mpmath.fsum(mpmath.exp(mpmath.mpf(float(v))) for v in z)
        return float(mpmath.mpf(float(z[t])) - mpmath.log(s)), float(mpmath.log(s))


def test_ref_matches_50_digit_direct_sum_on_tiny():
    w = datagen.tiny()
    logits, targets = w.generate()
    for i in range(w.n_rows):
        z = f32(logits[i, :w.vocab_real]).astype(np.float64) / 1.0
        for t in [int(targets[i]), 0, 999, int(np.argmax(z))]:
            ref, lse = O.ref_logp_row(logits[i], w.vocab_real, 1.0, t)
            want, want_lse = _mp_ref(z, t)
            assert abs(ref - want) < 1e-12
            assert abs(lse - want_lse) < 1e-12


@pytest.mark.parametrize("temperature", [0.7, 1.3])
def test_ref_matches_50_digit_direct_sum_small_rows(temperature):
    w = datagen.small(77, 3, 512, 509, sigma=2.5, temperature=temperature)
    logits, targets = w.generate()
    for i in range(3):
        x = f32(logits[i, :509])
        z = [_nearest_f32(Fraction(float(v)) / Fraction(float(np.float32(temperature)))) for v in x]
        ref, _ = O.ref_logp_row(logits[i], 509, temperature, int(targets[i]))
        want, _ = _mp_ref(z, int(targets[i]))
        assert abs(ref - want) < 1e-12


def test_all_equal_logits_give_minus_log_vocab():
    row = np.full(1024, bf16([1.5])[0], dtype=np.uint16)
    row[1000:] = datagen.BF16_NEG_INF
    for t in [0, 17, 999]:
        ref, lse = O.ref_logp_row(row, 1000, 0.7, t)
        assert abs(ref - (-6.907755278982137)) < 1e-14
        z = float(np.float32(1.5) / np.float32(0.7))
        assert abs(lse - (z + math.log(1000))) < 1e-13


@pytest.mark.parametrize("a,b", [(2.0, 1.0), (0.0, -3.5), (10.0, 10.0), (-1.25, 7.0)])
def test_two_token_closed_form(a, b):
    row = bf16([a, b])
    for temperature in (1.0, 0.5, 2.0):   # powers of two: the division is exact
        za, zb = a / temperature, b / temperature
        ref0, _ = O.ref_logp_row(row, 2, temperature, 0)
        ref1, _ = O.ref_logp_row(row, 2, temperature, 1)
        assert abs(ref0 - (-math.log1p(math.exp(zb - za)))) < 1e-14
        assert abs(ref1 - (-math.log1p(math.exp(za - zb)))) < 1e-14


def test_probabilities_sum_to_one_over_every_target():
    w = datagen.tiny()
    logits, _ = w.generate()
    for i in range(w.n_rows):
        refs = [O.ref_logp_row(logits[i], 1000, 1.0, t)[0] for t in range(1000)]
        assert abs(math.fsum(math.exp(r) for r in refs) - 1.0) < 1e-13


def test_ref_matches_torch_float64_log_softmax():
    import torch
    for w in (datagen.tiny(), datagen.full(n_rows=2)):
        logits, targets = w.generate()
        for i in range(w.n_rows):
            x = f32(logits[i, :w.vocab_real])
            z = (x / np.float32(w.temperature[i])).astype(np.float64)
            ls = torch.log_softmax(torch.from_numpy(z), dim=0).numpy()
            for t in [int(targets[i]), 0, w.vocab_real - 1]:
                ref, _ = O.ref_logp_row(logits[i], w.vocab_real, float(w.temperature[i]), t)
                assert abs(ref - ls[t]) < 1e-11


def test_shard_summary_merge_equals_direct_lse():
    """The per-shard (max, sum-exp) summaries over 8 canonical shards, merged left
    to right, reach the same log-sum-exp (page "Reproduce and profile the
    Qwen3-8B TP4/CP2 experiment", canonical virtual TP partition section)."""
    w = datagen.tiny()
    logits, targets = w.generate()
    shard = w.vocab_padded // 8
    for i in range(w.n_rows):
        z = f32(logits[i, :w.vocab_real]).astype(np.float64)
        ms, ls = [], []
        for s in range(8):
            seg = z[s * shard: min((s + 1) * shard, w.vocab_real)]
            m = seg.max()
            ms.append(m)
            ls.append(math.fsum(np.exp(seg - m).tolist()))
        M = max(ms)
        L = 0.0
        for m, l in zip(ms, ls):
            L = L + l * math.exp(m - M)
        _, lse = O.ref_logp_row(logits[i], w.vocab_real, 1.0, int(targets[i]))
        assert abs((M + math.log(L)) - lse) < 1e-13


def test_pad_columns_are_ignored_whatever_they_hold():
    base = datagen.small(91, 2, 1024, 1000, sigma=3.0, temperature=0.7)
    logits, targets = base.generate()
    want = [O.ref_logp_row(logits[i], 1000, 0.7, int(targets[i]))[0] for i in range(2)]
    for fill in (datagen.BF16_NAN, datagen.BF16_POS_INF, datagen.BF16_MAX_FINITE, 0x3F80):
        poisoned = logits.copy()
        poisoned[:, 1000:] = fill
        got = [O.ref_logp_row(poisoned[i], 1000, 0.7, int(targets[i]))[0] for i in range(2)]
        assert got == want


def test_neg_inf_logits_carry_zero_mass():
    vals = np.array([1.0, -2.0, 0.5, 3.0, -1.0], dtype=np.float32)
    row = bf16(vals)
    row_inf = bf16(np.array([1.0, -2.0, -np.inf, 3.0, -np.inf], dtype=np.float32))
    reduced = [1.0, -2.0, 3.0]
    for t, rt in ((0, 0), (1, 1), (3, 2)):
        ref, _ = O.ref_logp_row(row_inf, 5, 1.0, t)
        want, _ = _mp_ref(reduced, rt)
        assert abs(ref - want) < 1e-14
    ref2, _ = O.ref_logp_row(row_inf, 5, 1.0, 2)
    assert ref2 == float("-inf")
    assert np.isfinite(O.ref_logp_row(row, 5, 1.0, 2)[0])


def test_invalid_rows_are_nan():
    row = bf16([1.0, 2.0, 3.0, 0.0])
    for t in (float("nan"), -1.0, float("inf"), -1e-30):
        assert all(math.isnan(v) for v in O.ref_logp_row(row, 4, t, 0))
    for tgt in (-1, 4, 100):
        assert math.isnan(O.ref_logp_row(row, 4, 1.0, tgt)[0])
    for bad in (datagen.BF16_NAN, datagen.BF16_POS_INF):
        r = row.copy()
        r[1] = bad
        assert math.isnan(O.ref_logp_row(r, 4, 1.0, 0)[0])
    allneg = np.full(4, datagen.BF16_NEG_INF, dtype=np.uint16)
    assert math.isnan(O.ref_logp_row(allneg, 4, 1.0, 0)[0])
    # invalid top-p / top-k: policy NaN, reference unaffected
    for p, k in ((0.0, -1), (1.5, -1), (float("nan"), -1), (0.9, 0), (0.9, -2), (0.9, 5)):
        pol, ref, _ = O.nucleus_row(row, 4, 1.0, p, k, 2)
        assert math.isnan(pol) and np.isfinite(ref)


# --------------------------------------------------------------------------- greedy and T -> 0

def test_temperature_to_zero_limit_and_greedy():
    vals = np.array([0.5, 2.0, -1.0, 1.75, 0.0, 1.0], dtype=np.float32)
    row = bf16(vals)
    x = f32(row)
    am = int(np.argmax(x))
    prev = -math.inf
    for temperature in (1e-1, 1e-2, 1e-3):
        ref, _ = O.ref_logp_row(row, 6, temperature, am)
        assert prev < ref <= 0.0
        prev = ref
        for j in range(6):
            if j == am:
                continue
            r, _ = O.ref_logp_row(row, 6, temperature, j)
            lead = -(float(x[am]) - float(x[j])) / temperature
            slack = 1e-6 * abs(lead)   # fp32 rounding of x / T
            # z_j - z_max - log(6) <= ref(j) <= z_j - z_max, and the gap closes as T -> 0
            assert lead - math.log(6) - slack <= r <= lead + slack
            if temperature == 1e-3:
                assert abs(r - lead) <= slack
    assert prev > -1e-30
    for j in range(6):
        g, lse = O.ref_logp_row(row, 6, 0.0, j)
        assert g == (0.0 if j == am else float("-inf"))
        assert math.isnan(lse)
        g2, _ = O.ref_logp_row(row, 6, -0.0, j)
        assert g2 == g


def test_greedy_ties_take_lowest_index_and_limit_is_log_ties():
    vals = np.array([0.5, 2.0, -1.0, 2.0, 0.0, 2.0], dtype=np.float32)
    row = bf16(vals)
    assert O.ref_logp_row(row, 6, 0.0, 1)[0] == 0.0
    assert O.ref_logp_row(row, 6, 0.0, 3)[0] == float("-inf")
    for j in (1, 3, 5):
        r, _ = O.ref_logp_row(row, 6, 1e-3, j)
        assert abs(r - (-math.log(3))) < 1e-12


# --------------------------------------------------------------------------- support (brute force)

def _upper_closed(sub, z):
    s = set(sub)
    return all((i in s) for j in s for i in range(len(z)) if z[i] >= z[j])


def _brute_support(z, p, k):
    """Kept token set by exhaustive enumeration over subsets with exact rational masses."""
    V = len(z)
    M = max(z)
    mass = [Fraction(math.exp(v - M)) for v in z]
    idx = range(V)
    if k == -1 or k >= V:
        sk = set(idx)
    else:
        best = max(sum(mass[j] for j in c) for c in itertools.combinations(idx, k))
        sk = set()
        for c in itertools.combinations(idx, k):
            if sum(mass[j] for j in c) == best:
                sk |= set(c)
    if p >= 1.0:
        return sk, None
    zk = sum(mass[j] for j in sk)
    target = Fraction(p) * zk
    best = None
    margin = None
    for r in range(1, len(sk) + 1):
        for c in itertools.combinations(sorted(sk), r):
            if _upper_closed(c, z) and sum(mass[j] for j in c) >= target:
                if best is None or len(c) < len(best):
                    best = c
    # distance of the closest upper set's mass to the threshold (for float-rounding guards)
    for r in range(1, len(sk) + 1):
        for c in itertools.combinations(sorted(sk), r):
            if _upper_closed(c, z):
                d = abs(float((sum(mass[j] for j in c) - target) / zk))
                margin = d if margin is None else min(margin, d)
    return set(best), margin


def test_support_matches_subset_enumeration():
    rng = np.random.default_rng(2024)
    palette = np.array([-2.0, -0.5, 0.0, 0.75, 1.0, 1.5, 2.5, 3.0], dtype=np.float32)
    checked = 0
    for case in range(250):
        V = int(rng.integers(2, 10))
        vals = rng.choice(palette, size=V) if case % 2 else rng.normal(0, 2, size=V).astype(np.float32)
        row = bf16(vals)
        temperature = float(rng.choice([0.7, 1.0, 1.3]))
        p = float(np.float32(rng.choice([rng.uniform(0.05, 0.999), 1.0, 0.5])))
        k = int(rng.choice([-1, int(rng.integers(1, V + 1))]))
        z = [float(v) for v in O.scale_fp32(f32(row), temperature)]
        keep, margin = _brute_support(z, p, k)
        if margin is not None and margin < 1e-12:
            continue
        for t in range(V):
            pol, ref, info = O.nucleus_row(row, V, temperature, p, k, t)
            if t in keep:
                if len(keep) == V:
                    assert pol == ref
                else:
                    with mpmath.workdps(40):
                        want = float(mpmath.mpf(z[t]) - mpmath.log(
                            mpmath.fsum(mpmath.exp(mpmath.mpf(z[j])) for j in keep)))
                    assert abs(pol - want) < 1e-12, (vals, p, k, t)
            else:
                assert pol == float("-inf"), (vals, p, k, t, keep)
            assert info.support_size == len(keep)
        checked += 1
    assert checked > 200


def test_topk_one_and_tiny_p_keep_the_argmax_class():
    vals = np.array([1.0, 3.0, 2.0, 3.0, -1.0, 3.0, 0.0], dtype=np.float32)
    row = bf16(vals)
    for p, k in ((1.0, 1), (1e-30, -1), (0.2, 1), (1e-6, 3)):
        for t in range(7):
            pol, _, _ = O.nucleus_row(row, 7, 0.7, p, k, t)
            if vals[t] == 3.0:
                assert abs(pol - (-math.log(3))) < 1e-14
            else:
                assert pol == float("-inf")


def test_disabled_support_returns_reference_bytes():
    w = datagen.tiny()
    logits, targets = w.generate()
    for i in range(w.n_rows):
        for p, k in ((1.0, -1), (1.0, 1000)):
            pol, ref, _ = O.nucleus_row(logits[i], 1000, 1.0, p, k, int(targets[i]))
            assert pol == ref


@pytest.mark.parametrize("p,k", [(0.9, -1), (0.95, 50), (1.0, 20), (0.5, 300)])
def test_policy_is_normalised_and_shift_is_constant(p, k):
    w = datagen.tiny()
    logits, _ = w.generate()
    for i in range(2):
        _, _, info = O.nucleus_row(logits[i], 1000, 1.0, p, k, 0, want_mask=True)
        support = np.flatnonzero(info.support_mask)
        outside = np.flatnonzero(~info.support_mask)
        pols, shifts = [], []
        for t in support.tolist():
            pol, ref, _ = O.nucleus_row(logits[i], 1000, 1.0, p, k, t)
            pols.append(pol)
            shifts.append(pol - ref)
        assert abs(math.fsum(math.exp(v) for v in pols) - 1.0) < 1e-12
        assert max(shifts) - min(shifts) < 1e-12 and min(shifts) >= 0.0
        for t in outside[:20].tolist():
            assert O.nucleus_row(logits[i], 1000, 1.0, p, k, t)[0] == float("-inf")


# --------------------------------------------------------------------------- generator pins

def test_bf16_rounding_matches_torch():
    import torch
    a = np.concatenate([RNG.normal(0, 3, size=20000).astype(np.float32),
                        np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38, -3.4e38, np.inf, -np.inf],
                                 dtype=np.float32)])
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(datagen.f32_to_bf16_bits(a), want)


def test_generator_is_reproducible_and_row_addressable():
    w = datagen.full(n_rows=300)
    a, ta = w.generate(rows=[5, 299, 0])
    b, tb = w.generate(rows=[0, 5, 299])
    assert np.array_equal(a[0], b[1]) and np.array_equal(a[1], b[2]) and np.array_equal(a[2], b[0])
    assert list(ta) == [tb[1], tb[2], tb[0]]
    full_a, full_t = w.generate(threads=4)
    assert np.array_equal(full_a[[5, 299, 0]], a) and list(full_t[[5, 299, 0]]) == list(ta)
    assert np.all(a[:, datagen.QWEN3_VOCAB_REAL:] == datagen.BF16_NEG_INF)


def test_generator_fingerprints():
    # Fingerprints of the generator's own output (regression pins for the inputs).
    assert datagen.tiny().checksum(range(4)) == TINY_SHA
    assert datagen.full(n_rows=3).checksum(range(3)) == FULL3_SHA


TINY_SHA = "5eb4269e6ff408ad43d8642e4f9144fca24cebb87b2f27bf8f3bd15d84ea349b"
FULL3_SHA = "f45fe8a8a96e9a5ee26172c1f73281115ba217f84eee5cf4cf459b5df99786ea"


def test_golden_snapshot_is_current():
    """tests/golden/tiny.json was written by tests/golden/make_golden.py from the
    oracle; a change to the oracle's arithmetic must regenerate it deliberately."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny.json")))
    w = datagen.tiny()
    logits, targets = w.generate()
    for r in g["rows"]:
        i = r["row"]
        assert r["target"] == int(targets[i])
        ref, lse = O.ref_logp_row(logits[i], 1000, 1.0, r["target"])
        assert ref == r["ref_logp"] and lse == r["lse"]
        for c in r["support"]:
            pol, ref2, info = O.nucleus_row(logits[i], 1000, 1.0, c["top_p"], c["top_k"], c["target"])
            assert pol == c["policy_logp"] and ref2 == c["ref_logp"]
            assert info.support_size == c["support_size"]


# --------------------------------------------------------------------------- support record (threshold, lse)

def test_support_threshold_and_lse_match_subset_enumeration():
    rng = np.random.default_rng(77)
    checked = 0
    for case in range(150):
        V = int(rng.integers(2, 9))
        row = bf16(rng.normal(0, 2, size=V).astype(np.float32))
        temperature = float(rng.choice([0.7, 1.0, 1.3]))
        p = float(np.float32(rng.choice([rng.uniform(0.05, 0.999), 1.0])))
        k = int(rng.choice([-1, int(rng.integers(1, V + 1))]))
        x = [float(v) for v in f32(row)]
        z = [float(v) for v in O.scale_fp32(f32(row), temperature)]
        keep, margin = _brute_support(z, p, k)
        if margin is not None and margin < 1e-12:
            continue
        _, _, info = O.nucleus_row(row, V, temperature, p, k, 0)
        want_thr = float("-inf") if len(keep) == V else min(x[j] for j in keep)
        assert info.threshold == want_thr
        with mpmath.workdps(40):
            want = float(mpmath.log(mpmath.fsum(mpmath.exp(mpmath.mpf(z[j])) for j in keep)))
        assert abs(info.lse_support - want) < 1e-12
        checked += 1
    assert checked > 100


# --------------------------------------------------------------------------- gradient

def _forward_mp(z, t_idx, keep, g_ref, g_pol, scale=None):
    """g_ref * ref + g_pol * pol at 50 digits, for a fixed support `keep`
    (the policy term is dropped when the target is outside it: pol is the
    constant -inf there). `scale` divides z first (x-space evaluation)."""
    zz = [mpmath.mpf(v) if scale is None else mpmath.mpf(v) / mpmath.mpf(scale) for v in z]
    lse = mpmath.log(mpmath.fsum(mpmath.exp(v) for v in zz))
    f = g_ref * (zz[t_idx] - lse)
    if g_pol != 0 and t_idx in keep:
        lse_s = mpmath.log(mpmath.fsum(mpmath.exp(zz[j]) for j in keep))
        f += g_pol * (zz[t_idx] - lse_s)
    return f


def _grad_cases(seed, n):
    rng = np.random.default_rng(seed)
    for case in range(n):
        V = int(rng.integers(2, 9))
        vals = rng.normal(0, 2, size=V).astype(np.float32)
        if case % 5 == 0:
            vals[int(rng.integers(V))] = -np.inf if V > 1 else vals[0]
        row = bf16(vals)
        if not np.isfinite(f32(row)).any():
            continue
        temperature = float(rng.choice([0.7, 1.0, 1.3]))
        p = float(np.float32(rng.choice([rng.uniform(0.05, 0.999), 1.0])))
        k = int(rng.choice([-1, int(rng.integers(1, V + 1))]))
        t_idx = int(rng.choice(np.flatnonzero(np.isfinite(f32(row)))))  # -inf targets: test_grad_sums_to_zero...
        g_ref = float(rng.choice([0.0, 1.0, -0.37]))
        g_pol = float(rng.choice([0.0, 0.8, -1.9]))
        if g_ref == 0.0 and g_pol == 0.0:
            g_ref = 1.0
        yield row, V, temperature, p, k, t_idx, g_ref, g_pol


def test_grad_matches_50_digit_central_differences():
    """d/dz_j of the forward at the float32 point z = fl32(x/T), by central
    differences at 50 digits with the support held fixed (it is piecewise
    constant), times dz/dx = 1/T."""
    checked = 0
    h = mpmath.mpf("1e-20")
    for row, V, temperature, p, k, t_idx, g_ref, g_pol in _grad_cases(31, 160):
        z = [float(v) for v in O.scale_fp32(f32(row), temperature)]
        keep, margin = _brute_support([v if np.isfinite(v) else -1e300 for v in z], p, k)
        if margin is not None and margin < 1e-12:
            continue
        got = O.grad_row(row, V + 3, V, temperature, t_idx, g_ref, g_pol, p, k)
        assert np.all(got[V:] == 0.0)
        with mpmath.workdps(50):
            for j in range(V):
                zp = list(z); zp[j] = mpmath.mpf(z[j]) + h
                zm = list(z); zm[j] = mpmath.mpf(z[j]) - h
                d = (_forward_mp(zp, t_idx, keep, g_ref, g_pol) - _forward_mp(zm, t_idx, keep, g_ref, g_pol)) / (2 * h)
                want = float(d) / float(np.float32(temperature))
                assert abs(got[j] - want) < 1e-12 * (1 + abs(want)), (row, temperature, p, k, t_idx, j, got[j], want)
        checked += 1
    assert checked > 100


def test_grad_in_x_space_carries_the_temperature_factor():
    """Differences of the forward in x itself (z = x/T at 50 digits, no float32
    rounding): agrees with the gradient up to the float32 rounding of z."""
    h = mpmath.mpf("1e-20")
    rng = np.random.default_rng(5)
    for _ in range(30):
        V = 6
        row = bf16(rng.normal(0, 2, size=V).astype(np.float32))
        x = [float(v) for v in f32(row)]
        for temperature in (0.5, 1.7):
            t_idx = int(rng.integers(V))
            got = O.grad_row(row, V, V, temperature, t_idx, 1.0, 0.0)
            with mpmath.workdps(50):
                for j in range(V):
                    xp = list(x); xp[j] = mpmath.mpf(x[j]) + h
                    xm = list(x); xm[j] = mpmath.mpf(x[j]) - h
                    T = float(np.float32(temperature))
                    d = (_forward_mp(xp, t_idx, set(), 1.0, 0.0, T) - _forward_mp(xm, t_idx, set(), 1.0, 0.0, T)) / (2 * h)
                    assert abs(got[j] - float(d)) < 1e-6 * (1 + abs(float(d)))


def test_grad_matches_torch_autograd_on_tiny_rows():
    import torch
    w = datagen.tiny()
    logits, targets = w.generate()
    for i in range(w.n_rows):
        for p, k, g_ref, g_pol in ((1.0, -1, 1.0, 0.0), (0.9, -1, 0.3, -1.2), (0.95, 50, -0.5, 2.0), (1.0, 20, 0.0, 1.0)):
            t_idx = int(targets[i]) if i % 2 else int(np.argmax(f32(logits[i][:1000])))
            pol, _, info = O.nucleus_row(logits[i], 1000, 1.0, p, k, t_idx, want_mask=True)
            z = torch.tensor(O.scale_fp32(f32(logits[i][:1000]), 1.0), dtype=torch.float64, requires_grad=True)
            f = g_ref * torch.log_softmax(z, 0)[t_idx]
            if np.isfinite(pol):
                mask = torch.from_numpy(info.support_mask)
                f = f + g_pol * (z[t_idx] - torch.logsumexp(z[mask], 0))
            f.backward()
            got = O.grad_row(logits[i], 1024, 1000, 1.0, t_idx, g_ref, g_pol, p, k)
            assert np.allclose(got[:1000], z.grad.numpy(), rtol=1e-12, atol=1e-15)
            assert np.all(got[1000:] == 0.0)


def test_grad_sums_to_zero_and_special_rows():
    w = datagen.tiny()
    logits, targets = w.generate()
    row, tg = logits[1], int(targets[1])
    for p, k in ((1.0, -1), (0.9, -1), (0.5, 7)):
        g = O.grad_row(row, 1024, 1000, 0.7, tg, 0.6, -1.4, p, k)
        assert abs(math.fsum(g.tolist())) < 1e-12 and np.all(np.isfinite(g))
    # zero upstream gradients: exact zeros, even for an invalid row
    assert np.all(O.grad_row(row, 1024, 1000, float("nan"), tg, 0.0, 0.0) == 0.0)
    # greedy rows: the logprob is piecewise constant
    assert np.all(O.grad_row(row, 1024, 1000, 0.0, tg, 1.0, 1.0, 0.9, 5) == 0.0)
    # invalid rows: NaN on the real columns, zeros on the pads
    for t, target in ((float("nan"), tg), (-1.0, tg), (1.0, 1000), (1.0, -1)):
        g = O.grad_row(row, 1024, 1000, t, target, 1.0)
        assert np.all(np.isnan(g[:1000])) and np.all(g[1000:] == 0.0)
    bad = row.copy(); bad[3] = 0x7FC0
    assert np.all(np.isnan(O.grad_row(bad, 1024, 1000, 1.0, tg, 0.0, 1.0)[:1000]))
    # invalid top-p: NaN only when the policy term is asked for
    assert np.all(np.isnan(O.grad_row(row, 1024, 1000, 1.0, tg, 1.0, 1.0, 1.5, -1)[:1000]))
    assert np.array_equal(O.grad_row(row, 1024, 1000, 1.0, tg, 1.0, 0.0, 1.5, -1), O.grad_row(row, 1024, 1000, 1.0, tg, 1.0))
    # target outside the support: the policy term vanishes
    _, _, info = O.nucleus_row(row, 1000, 1.0, 0.5, 3, 0, want_mask=True)
    outside = int(np.flatnonzero(~info.support_mask)[0])
    assert np.array_equal(O.grad_row(row, 1024, 1000, 1.0, outside, 0.7, 5.0, 0.5, 3),
                          O.grad_row(row, 1024, 1000, 1.0, outside, 0.7, 0.0))
    # a -inf target: its logprob is -inf but d/dx_t = (1 - p_t) / T = 1 / T, the rest -p_j / T (sum 0)
    neg = row.copy(); neg[9] = datagen.BF16_NEG_INF
    g = O.grad_row(neg, 1024, 1000, 2.0, 9, 1.0)
    assert g[9] == 0.5 and abs(math.fsum(g.tolist())) < 1e-12
    # ... and the same holds for the policy term when the support is the whole
    # vocabulary (the -inf target is then inside it), while a restricted
    # support leaves the -inf target outside: no policy term
    assert np.array_equal(O.grad_row(neg, 1024, 1000, 2.0, 9, 0.0, 1.0), g)
    assert np.all(O.grad_row(neg, 1024, 1000, 2.0, 9, 0.0, 1.0, 0.9) == 0.0)
    # disabled support: the policy term equals the reference term
    a = O.grad_row(row, 1024, 1000, 1.3, tg, 0.25, 0.5)
    b = O.grad_row(row, 1024, 1000, 1.3, tg, 0.75, 0.0)
    assert np.allclose(a, b, rtol=1e-14, atol=1e-18)

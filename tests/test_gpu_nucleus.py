"""GPU parity of rlk_logp_nucleus (policy over the top-k-then-top-p support and
the full-vocabulary reference) against the CPU oracle.

Defining passages: RL-Kernel page "Configurable H100 consistency runs":
sampling paragraph (top-p in (0, 1], top-k -1 or up to the real vocabulary,
support from the real vocabulary, per-request temperatures), mode/KL paragraph
(the policy keeps its top-p/top-k support, the KL reference is the
full-vocabulary temperature-scaled logprob), command examples (top-k
independent of top-p and temperature).

Rows whose top-p decision lies within 2e-6 of p (the ambiguity band) may match
the oracle under either neighbouring cut; every other row must match its
support exactly and its value within 2e-5.
"""
import math

import numpy as np
import pytest

import datagen
import invariant_token_log_fp32_amd as rlk
from oracle import logp as O

from gpu_util import (TOL, WINDOW_MAG_LO, WINDOW_N_MAG, assert_close, assert_nucleus_close, exact_reference_rows,
                      report, row_tolerance, say, to_host, upload, upload_logits)

pytestmark = pytest.mark.gpu

GROUPS = (1, 2, 4, 8)


def run_nucleus(logits_np, vr, temps, top_p, top_k, targets, groups=1, vp=None):
    import torch
    lg = upload_logits(logits_np)
    pol, ref = rlk.logp_nucleus(lg, upload(temps, torch.float32), upload(top_p, torch.float32),
                                upload(top_k, torch.int32), upload(targets, torch.int64),
                                vocab_real=vr, vocab_padded=vp, groups=groups)
    full = rlk.logp_full(lg, upload(temps, torch.float32), upload(targets, torch.int64), vocab_real=vr,
                         vocab_padded=vp, groups=groups)
    torch.cuda.synchronize()
    return to_host(pol), to_host(ref), to_host(full)


def check_ref_against_full(ref, full, logits, vr, temps, top_p, top_k, targets, tol, what):
    """The nucleus reference against rlk_logp_full's on every row: the same
    bytes where both come from the float32 shard sums, within the tolerance
    where the nucleus reference comes from the exact class masses."""
    exact = exact_reference_rows(logits, vr, temps, top_p, top_k, targets)
    assert ref[~exact].tobytes() == full[~exact].tobytes(), f"{what}: float32-reference rows differ from rlk_logp_full"
    tol = np.broadcast_to(np.asarray(tol, dtype=np.float64), ref.shape)
    err = assert_close(ref[exact], full[exact], tol=tol[exact], what=f"{what}: exact-mass reference vs rlk_logp_full")
    report(f"{what}: {int(exact.sum())} exact-mass reference rows, largest |ref - full| {err:.2e}")


def check(logits, vr, temps, top_p, top_k, targets, what, vp=None, groups_list=GROUPS, extra_tol=0.0):
    want_pol, want_ref, infos = O.nucleus_logp(logits, vr, temps, top_p, top_k, targets)
    tol = row_tolerance(logits, vr, temps) + extra_tol
    float_ref = ~exact_reference_rows(logits, vr, temps, top_p, top_k, targets)
    first = None
    first_ref = None
    for groups in groups_list:
        pol, ref, full = run_nucleus(logits, vr, temps, top_p, top_k, targets, groups, vp)
        assert ref[float_ref].tobytes() == full[float_ref].tobytes(), \
            f"{what}: reference bytes of the float32-reference rows differ from rlk_logp_full"
        assert_close(ref, want_ref, tol=tol, what=f"{what} ref g{groups}")
        if first_ref is None:
            first_ref = ref.tobytes()
        assert ref.tobytes() == first_ref, f"{what}: reference bytes differ between groups"
        n_amb, n_alt = assert_nucleus_close(pol, want_pol, infos, tol=tol, what=f"{what} policy g{groups}")
        if n_amb:
            report(f"{what} g{groups}: {n_amb} rows in the ambiguity band, {n_alt} matched a neighbouring cut")
        if first is None:
            first = pol.tobytes()
        assert pol.tobytes() == first, f"{what}: policy bytes differ between groups"
    return want_pol, infos


def support_targets(logits, vr, temps, top_p, top_k, seed):
    """Targets drawn uniformly from each row's oracle support."""
    rng = np.random.default_rng(seed)
    out = np.empty(logits.shape[0], dtype=np.int64)
    for i in range(logits.shape[0]):
        _, _, info = O.nucleus_row(logits[i], vr, float(temps[i]), float(top_p[i]), int(top_k[i]), 0,
                                   want_mask=True)
        idx = np.flatnonzero(info.support_mask)
        out[i] = int(rng.choice(idx))
    return out


CASES = [(0.9, -1), (0.95, 50), (1.0, 10), (0.5, 3), (0.99, 128), (1e-6, -1), (1.0, 1), (0.3, 1000),
         (1.0, 999), (0.999, -1)]


def test_tiny_every_target_all_cases():
    say("case: tiny nucleus, every target")
    w = datagen.tiny()
    logits, _ = w.generate()
    rep = np.repeat(logits, 1000, axis=0)
    tg = np.tile(np.arange(1000), 4)
    n = rep.shape[0]
    temps = np.ones(n, dtype=np.float32)
    for p, k in CASES:
        top_p = np.full(n, p, dtype=np.float32)
        top_k = np.full(n, k, dtype=np.int32)
        want_pol, _ = check(rep, 1000, temps, top_p, top_k, tg, f"tiny p={p} k={k}", groups_list=(1, 8))
        pol, _, _ = run_nucleus(rep, 1000, temps, top_p, top_k, tg)
        for i in range(4):
            blk = pol[i * 1000:(i + 1) * 1000].astype(np.float64)
            fin = np.isfinite(blk)
            assert abs(math.fsum(np.exp(blk[fin])) - 1.0) < 3e-5
            assert np.array_equal(fin, np.isfinite(want_pol[i * 1000:(i + 1) * 1000]))


def _palette_rows(seed, n, vp, vr):
    """Rows drawn from a few BF16 values: large tie classes at every boundary."""
    rng = np.random.default_rng(seed)
    pal = np.array([-3.0, -1.0, -0.5, 0.0, 0.25, 1.0, 1.5, 2.0, 2.5, 3.0], dtype=np.float32)
    rows = np.full((n, vp), datagen.BF16_NEG_INF, dtype=np.uint16)
    for i in range(n):
        rows[i, :vr] = datagen.f32_to_bf16_bits(rng.choice(pal, size=vr))
    return rows


def test_tied_classes_and_parameter_mix():
    say("case: ties and parameter mix")
    vp, vr = 2048, 1999
    logits = _palette_rows(5, 40, vp, vr)
    rng = np.random.default_rng(6)
    temps = rng.choice(np.array([0.7, 1.0, 1.3, 0.4], dtype=np.float32), 40)
    top_p = rng.choice(np.array([0.95, 0.99, 0.5, 1.0, 0.1], dtype=np.float32), 40)
    top_k = rng.choice(np.array([-1, 128, 1, 300, 1999, 1500], dtype=np.int32), 40)
    targets = rng.integers(0, vr, 40)
    check(logits, vr, temps, top_p, top_k, targets, "ties")
    targets = support_targets(logits, vr, temps, top_p, top_k, 8)
    check(logits, vr, temps, top_p, top_k, targets, "ties in-support")


def test_tied_classes_without_zero():
    """Palette rows with no zero and no value below 2^-24 in magnitude: every
    row stays in the 16-bit rank window, so the ties are resolved there."""
    say("case: ties without zero")
    vp, vr = 2048, 1999
    rng = np.random.default_rng(61)
    pal = np.array([-3.0, -1.0, -0.5, 0.25, 1.0, 1.5, 2.0, 2.5, 3.0], dtype=np.float32)
    n = 40
    logits = np.full((n, vp), datagen.BF16_NEG_INF, dtype=np.uint16)
    for i in range(n):
        logits[i, :vr] = datagen.f32_to_bf16_bits(rng.choice(pal, size=vr))
    temps = rng.choice(np.array([0.7, 1.0, 1.3, 0.4], dtype=np.float32), n)
    top_p = rng.choice(np.array([0.95, 0.99, 0.5, 1.0, 0.1], dtype=np.float32), n)
    top_k = rng.choice(np.array([-1, 128, 1, 300, 1999, 1500], dtype=np.int32), n)
    targets = support_targets(logits, vr, temps, top_p, top_k, 62)
    check(logits, vr, temps, top_p, top_k, targets, "ties without zero")


def test_top_p_near_one_and_edges():
    """Top-p values just below 1 (the threshold ceil(p * Z) then lies within a
    few tokens' mass of the total), a tiny top-p (the argmax class) and mid
    values, with top-k off, on rows of 8 shards of 2400 columns and the
    benchmark's value distribution, with and without a spike."""
    say("case: top-p near 1 and edges")
    vp, vr = 19200, 19137
    n = 48
    rng = np.random.default_rng(71)
    logits = np.full((n, vp), datagen.BF16_NEG_INF, dtype=np.uint16)
    for i in range(n):
        bits, _, _ = datagen.row_values((71, i), vr, 2.5, 8.0 if i % 2 else None)
        logits[i, :vr] = bits
    p_vals = np.array([np.nextafter(np.float32(1), np.float32(0)), 1 - 2.0 ** -20, 0.9999, 0.999, 0.99, 0.95,
                       0.5, 1e-7], dtype=np.float32)
    top_p = p_vals[np.arange(n) % len(p_vals)]
    temps = np.array([0.7, 1.3, 1.0], dtype=np.float32)[(np.arange(n) // len(p_vals)) % 3]
    top_k = np.full(n, -1, dtype=np.int32)
    targets = support_targets(logits, vr, temps, top_p, top_k, 72)
    check(logits, vr, temps, top_p, top_k, targets, "top-p near 1", groups_list=(1, 8))
    # targets just outside the support of the rows whose support is not everything
    targets = rng.integers(0, vr, size=n).astype(np.int64)
    check(logits, vr, temps, top_p, top_k, targets, "top-p near 1, uniform targets", groups_list=(1, 8))


def test_deep_top_p_scans():
    """Rows whose probability mass spreads over most of the support window, so
    that the top-p crossing lies many 256-class steps below the maximum: the
    values are +-2^U(-24, 3) (a few zeros in every other row), at temperatures
    2 and 8 where the masses of all tokens are within a small factor of each
    other. The p grid puts the crossing in many different steps, with top-k off
    and on (k = 12000, so the top-p threshold comes from the exact top-k
    mass)."""
    say("case: deep top-p scans")
    vp, vr = 19200, 19137
    p_grid = np.array([0.05, 0.2, 0.35, 0.5, 0.65, 0.8, 0.95, 0.999], dtype=np.float32)
    rows, T, P, K = [], [], [], []
    rng = np.random.default_rng(83)
    for temp in (2.0, 8.0):
        for k in (-1, 12000):
            for i, p in enumerate(p_grid):
                r = np.full(vp, datagen.BF16_NEG_INF, dtype=np.uint16)
                mag = np.exp2(rng.uniform(-24.0, 3.0, vr)).astype(np.float32)
                sign = np.where(rng.random(vr) < 0.5, -1.0, 1.0).astype(np.float32)
                r[:vr] = datagen.f32_to_bf16_bits(mag * sign)
                if i % 2:
                    r[rng.integers(0, vr, 5)] = 0
                rows.append(r)
                T.append(temp)
                P.append(p)
                K.append(k)
    logits = np.stack(rows)
    temps = np.array(T, np.float32)
    top_p = np.array(P, np.float32)
    top_k = np.array(K, np.int32)
    targets = support_targets(logits, vr, temps, top_p, top_k, 84)
    check(logits, vr, temps, top_p, top_k, targets, "deep top-p scans", groups_list=(1, 8))


def test_classes_of_millions_of_tokens():
    """Rows of 10,000,000 columns where one class holds 6 to 10 million tokens,
    so a class mass count * weight has a high part above 2^31 (the widest the
    search's integer masses get below the 2^24-token limit): all tokens equal
    (top-k 5 keeps the whole tied class), and 60% of the tokens on the maximum
    with the rest spread below (top-p 0.5 and 0.9)."""
    say("case: classes of millions of tokens")
    vp = vr = 10_000_000
    rng = np.random.default_rng(97)
    rows, T, P, K = [], [], [], []
    eq = np.full(vp, datagen.f32_to_bf16_bits(np.array([3.0], np.float32))[0], dtype=np.uint16)
    rows.append(eq)
    T.append(0.7)
    P.append(1.0)
    K.append(5)
    for p in (0.5, 0.9):
        r = datagen.f32_to_bf16_bits(rng.normal(0.0, 1.0, vp).astype(np.float32))
        r[rng.random(vp) < 0.6] = datagen.f32_to_bf16_bits(np.array([6.0], np.float32))[0]
        rows.append(r)
        T.append(1.0)
        P.append(p)
        K.append(-1)
    logits = np.stack(rows)
    temps = np.array(T, np.float32)
    top_p = np.array(P, np.float32)
    top_k = np.array(K, np.int32)
    targets = np.array([123, int(np.argmax(datagen.bf16_bits_to_f32(rows[1]))), 7], dtype=np.int64)
    # the float32 shard sums of the reference add one rounding per term of an
    # accumulator: 2441 terms here against 38 at the benchmark's vocabulary, so
    # the reference (and a policy equal to it) gets that many 2^-24 more
    depth = (vp // 8 // 8 + 64) // 64 + 1 + 3 + 6
    check(logits, vr, temps, top_p, top_k, targets, "classes of millions of tokens", vp=vp, groups_list=(1, 8),
          extra_tol=depth * 2.0 ** -24)


def test_row_maximum_beyond_the_search_range():
    """The support search covers rows whose largest scaled logit has
    |max x * log2(e) / T| < 2^20. At T 0.05 a maximum of 35840 (2^20 - 14k)
    is inside and is compared with the oracle; 37120, and a row of -40000
    everywhere, are beyond it: policy NaN, status -1, the reference as usual.
    Both the window path and the general path (a 1e-9 logit in the row) are
    covered."""
    import torch
    say("case: row maximum beyond the search range")
    vp, vr = 3072, 3000
    rng = np.random.default_rng(99)
    base = datagen.f32_to_bf16_bits(rng.normal(0.0, 2.5, vr).astype(np.float32))
    tiny = datagen.f32_to_bf16_bits(np.array([1e-9], np.float32))[0]
    rows, inside = [], []
    for top in (35840.0, 37120.0):
        for general in (False, True):
            r = np.full(vp, datagen.BF16_NEG_INF, dtype=np.uint16)
            r[:vr] = base
            r[17] = datagen.f32_to_bf16_bits(np.array([top], np.float32))[0]
            if general:
                r[29] = tiny
            rows.append(r)
            inside.append(top == 35840.0)
    r = np.full(vp, datagen.BF16_NEG_INF, dtype=np.uint16)
    r[:vr] = datagen.f32_to_bf16_bits(np.array([-40000.0], np.float32))[0]
    rows.append(r)
    inside.append(False)
    logits = np.stack(rows)
    n = logits.shape[0]
    temps = np.full(n, 0.05, np.float32)
    top_p = np.full(n, 0.9, np.float32)
    top_k = np.full(n, -1, np.int32)
    targets = np.full(n, 17, np.int64)
    inside = np.array(inside)
    c = np.float32(np.float32(1.4426950408889634) / np.float32(0.05))
    for i in range(n):
        m = float(datagen.bf16_bits_to_f32(logits[i, :vr]).max())
        assert (abs(float(np.float32(np.float32(m) * c))) < 2.0 ** 20) == inside[i]
    want_pol, want_ref, infos = O.nucleus_logp(logits, vr, temps, top_p, top_k, targets)
    tol = row_tolerance(logits, vr, temps)
    lg = upload_logits(logits)
    for groups in (1, 8):
        pol, ref, lse, state = rlk.logp_nucleus(lg, upload(temps, torch.float32), upload(top_p, torch.float32),
                                                upload(top_k, torch.int32), upload(targets, torch.int64),
                                                vocab_real=vr, groups=groups, return_state=True)
        torch.cuda.synchronize()
        pol, ref, state = to_host(pol), to_host(ref), to_host(state)
        assert_close(ref, want_ref, tol=tol, what=f"search range ref g{groups}")
        assert np.all(np.isnan(pol[~inside])), pol
        assert np.all(state[~inside, 2] == -1), state
        assert_nucleus_close(pol[inside], want_pol[inside], [infos[i] for i in np.flatnonzero(inside)],
                             tol=tol[inside], what=f"search range policy g{groups}")


# BF16 patterns at and just past the ends of the support window's value
# ranges: the top (4080 is the largest magnitude inside, 4096 and the next
# value outside, both signs), the smallest magnitudes (2^-24 inside, the next
# smaller value outside, both signs), +-0 (a class of the window), large
# negative values (-4.24e9 / -4.26e9 and -1.823e19 / -1.830e19, outside), and
# values inside it around +-256.
EDGE_BITS = [0x4380, 0x4381, 0xC37D, 0xC37E, 0x437E, 0x3380, 0x337F, 0xB380, 0xB37F,
             0x457F, 0x4580, 0x4581, 0xC57F, 0xC580, 0x0000, 0x8000,
             0xCF7D, 0xCF7E, 0xDF7D, 0xDF7E]
OUTSIDE_WINDOW = {0x337F, 0xB37F, 0x4580, 0x4581, 0xC580, 0xCF7D, 0xCF7E, 0xDF7D, 0xDF7E}


def test_window_edge_values():
    """Rows holding one value at or just past an edge of the rank window, with
    supports that reach that value (top-k down to the last classes, top-p 1)
    or stop above it; targets on that value and on the maximum."""
    say("case: window edge values")
    vp, vr = 3072, 3000
    rng = np.random.default_rng(71)
    rows, T, P, K, TG = [], [], [], [], []
    for bits in EDGE_BITS:
        for p, k in ((0.9, -1), (1.0, vr - 1), (1.0, vr), (0.5, 3), (0.999, vr - 2)):
            for tg_edge in (True, False):
                r = np.full(vp, datagen.BF16_NEG_INF, dtype=np.uint16)
                r[:vr] = datagen.f32_to_bf16_bits(rng.normal(0.0, 2.5, vr).astype(np.float32))
                col = int(rng.integers(0, vr))
                r[col] = bits
                rows.append(r)
                T.append(0.7)
                P.append(p)
                K.append(k)
                TG.append(col if tg_edge else int(np.argmax(datagen.bf16_bits_to_f32(r[:vr]))))
    logits = np.stack(rows)
    check(logits, vr, np.array(T, np.float32), np.array(P, np.float32), np.array(K, np.int32),
          np.array(TG, np.int64), "window edges")


def window_rank_bits(r):
    """BF16 pattern of the window class at rank r in value order: positive
    magnitudes from the largest down, then +-0, then negative magnitudes from
    the smallest up."""
    n = WINDOW_N_MAG
    if r < n:
        return WINDOW_MAG_LO + (n - 1 - r)
    if r == n:
        return 0
    return 0x8000 | (WINDOW_MAG_LO + (r - n - 1))


def test_row_maximum_in_every_step():
    """Rows whose maximum is the first or the last class of each 256-class
    step of the window (the kernel's row-maximum scan and step totals work in
    these steps; the eight wavefronts scan the first 32 steps in parallel and a
    row whose every token is at most -4 has its maximum in the steps scanned
    after them), the other tokens drawn from the classes below the maximum,
    ties of the maximum included (in one row the zero class holds only -0);
    top-p 0.9 alone and top-p 0.95 with top-k 50."""
    n_mag = WINDOW_N_MAG
    last = 2 * n_mag
    starts = [256 * s for s in range(n_mag // 256)] + [n_mag] + [n_mag + 1 + 256 * s for s in range(n_mag // 256)]
    maxima = sorted({r for s0 in starts for r in (s0, s0 if s0 == n_mag else s0 + 255)})
    assert maxima[-1] == last and len(maxima) == 4 * (n_mag // 256) + 1
    vp, vr = 2048, 2000
    rng = np.random.default_rng(77)
    rows, T, P, K = [], [], [], []
    for t, p, k in ((1.0, 0.9, -1), (0.7, 0.95, 50)):
        for r in maxima:
            ranks = rng.integers(r + 1, min(r + 1500, last) + 1, size=vr) if r < last else np.full(vr, r)
            top = rng.choice(vr, 3, replace=False)
            ranks[top] = r
            row = np.full(vp, datagen.BF16_NEG_INF, dtype=np.uint16)
            row[:vr] = np.array([window_rank_bits(int(q)) for q in ranks], dtype=np.uint16)
            if r == n_mag and k != -1:
                row[top] = 0x8000  # the zero class as -0 only: the maximum is not a non-negative pattern
            rows.append(row)
            T.append(t)
            P.append(p)
            K.append(k)
    logits = np.stack(rows)
    temps, top_p, top_k = np.array(T, np.float32), np.array(P, np.float32), np.array(K, np.int32)
    tg = support_targets(logits, vr, temps, top_p, top_k, 78)
    tg[::5] = rng.integers(0, vr, size=len(tg[::5]))  # some targets outside the support
    assert exact_reference_rows(logits, vr, temps, top_p, top_k, tg).all()
    say(f"case: row maximum in every window step ({len(rows)} rows)")
    check(logits, vr, temps, top_p, top_k, tg, "maximum in every step")


def test_support_limited_rows_match_enumeration():
    """Rows with at most 12 finite real logits (the rest -inf): the oracle's
    support on these is pinned by exhaustive subset enumeration."""
    say("case: support-limited rows")
    vp, vr = 1024, 1000
    rng = np.random.default_rng(12)
    n = 64
    logits = np.full((n, vp), datagen.BF16_NEG_INF, dtype=np.uint16)
    for i in range(n):
        m = int(rng.integers(1, 13))
        cols = rng.choice(vr, m, replace=False)
        vals = rng.choice(np.array([0.0, 0.5, 1.0, 1.25, 2.0, -1.0], np.float32), m)
        logits[i, cols] = datagen.f32_to_bf16_bits(vals)
    temps = rng.choice(np.array([0.7, 1.0, 1.3], np.float32), n)
    top_p = rng.choice(np.array([0.3, 0.6, 0.9, 1.0], np.float32), n)
    top_k = rng.choice(np.array([-1, 1, 2, 3, 5], np.int32), n)
    targets = support_targets(logits, vr, temps, top_p, top_k, 13)
    check(logits, vr, temps, top_p, top_k, targets, "support-limited")


def test_special_rows():
    say("case: nucleus special rows")
    vp, vr = 4096, 4000
    rng = np.random.default_rng(21)
    base = datagen.f32_to_bf16_bits(rng.normal(0, 2.5, vr).astype(np.float32))
    rows, T, P, K, TG = [], [], [], [], []

    def add(t, p, k, tg, row=base):
        r = np.full(vp, datagen.BF16_NEG_INF, dtype=np.uint16)
        r[:vr] = row
        rows.append(r)
        T.append(t)
        P.append(p)
        K.append(k)
        TG.append(tg)

    am = int(np.argmax(datagen.bf16_bits_to_f32(base)))
    for p, k in ((0.0, -1), (1.5, -1), (float("nan"), -1), (0.9, 0), (0.9, -2), (0.9, vr + 1)):
        add(0.7, p, k, am)                   # invalid top-p / top-k: policy NaN, reference valid
    add(0.0, 0.9, 5, am)                     # greedy
    add(0.0, 0.9, 5, am + 1)
    add(0.7, 1.0, -1, 3)                     # disabled: policy == reference
    add(0.7, 1.0, vr, 3)
    add(0.7, 1.0, vr - 1, 3)                 # top-k keeps all but the minimum class
    add(0.7, 0.9, -1, 3, row=np.full(vr, datagen.f32_to_bf16_bits(np.float32([1.0]))[0], np.uint16))  # all equal
    add(float("nan"), 0.9, 5, 3)
    add(0.7, 0.9, 5, -4)
    add(0.7, 0.9, -1, vr)                    # target past the real columns
    # rows a search would take whose reference cannot come from the window's masses: no finite
    # token, a NaN or a +inf logit (both outputs NaN), a huge finite logit (general path)
    add(0.7, 0.9, -1, 3, row=np.full(vr, datagen.BF16_NEG_INF, np.uint16))
    for bad in (datagen.BF16_NAN, datagen.BF16_POS_INF, datagen.f32_to_bf16_bits(np.float32([70000.0]))[0]):
        r = base.copy()
        r[17] = bad
        add(0.7, 0.9, -1, 3, row=r)
        add(1.3, 0.95, 128, 17, row=r)
    logits = np.stack(rows)
    check(logits, vr, np.array(T, np.float32), np.array(P, np.float32), np.array(K, np.int32),
          np.array(TG, np.int64), "special")


@pytest.fixture(scope="module")
def qwen_logits():
    w = datagen.nucleus()
    say("generating the 8192 x 152576 workload")
    logits, targets = w.generate()
    return w, logits, targets


def general_path_rows(logits, vocab_real, chunk=512, zeros=False):
    """Rows that the kernel sends to its general path, found from the BF16 bits:
    a real token other than -inf and +-0 whose magnitude is below 2^-24 or at
    least 4096 (NaN and +-inf included). With `zeros`, also the rows holding a
    +-0, which the window's zero class takes."""
    out = []
    for r0 in range(0, logits.shape[0], chunk):
        b = logits[r0:r0 + chunk, :vocab_real]
        mag = b & np.uint16(0x7FFF)
        outside = ((mag < np.uint16(0x3380)) | (mag >= np.uint16(0x4580))) & (mag != 0) & (b != np.uint16(0xFF80))
        if zeros:
            outside |= mag == 0
        hit = outside.any(axis=1)
        out.extend((np.flatnonzero(hit) + r0).tolist())
    return np.array(out, dtype=np.int64)


def test_general_path_row_predicate():
    """The host predicate above on values at and past each end of the window."""
    vr = 16
    rows = np.full((len(EDGE_BITS), vr), datagen.f32_to_bf16_bits(np.float32([1.0]))[0], dtype=np.uint16)
    for i, b in enumerate(EDGE_BITS):
        rows[i, 3] = b
    rows[0, 5] = datagen.BF16_NEG_INF
    got = set(general_path_rows(rows, vr).tolist())
    assert got == {i for i, b in enumerate(EDGE_BITS) if b in OUTSIDE_WINDOW}
    got = set(general_path_rows(rows, vr, zeros=True).tolist())
    assert got == {i for i, b in enumerate(EDGE_BITS) if b in OUTSIDE_WINDOW or b in (0, 0x8000)}


def compare_rows(logits, w, tg, pol, ref, rows, what):
    want_pol, want_ref, infos = O.nucleus_logp(logits[rows], w.vocab_real, w.temperature[rows], w.top_p[rows],
                                               w.top_k[rows], tg[rows])
    assert_close(ref[rows], want_ref, tol=row_tolerance(logits[rows], w.vocab_real, w.temperature[rows]),
                 what=f"{what} ref")
    n_amb, n_alt = assert_nucleus_close(pol[rows], want_pol, infos,
                                        tol=row_tolerance(logits[rows], w.vocab_real, w.temperature[rows]),
                                        what=f"{what} policy")
    report(f"{what}: {len(rows)} rows, {n_amb} in the ambiguity band, {n_alt} matched a neighbouring cut")
    return n_amb, n_alt


def test_full_size_nucleus_sampled(qwen_logits):
    """8192 x 152576, T = 0.7, top-p 0.95, top-k off, in the benchmark's launch
    configuration: 40 sampled rows and every row holding a zero (the window's
    zero class) or a token outside the window (the general path) get targets
    from their oracle nucleus; every row's reference is checked against
    rlk_logp_full's. No sampled row may match only a neighbouring top-p cut."""
    w, logits, targets = qwen_logits
    rows = np.random.default_rng(3003).choice(w.n_rows, 40, replace=False)
    gen = general_path_rows(logits, w.vocab_real, zeros=True)
    report(f"nucleus full: {len(general_path_rows(logits, w.vocab_real))} general-path rows, "
           f"{len(gen)} rows with a zero or a token outside the window")
    assert len(gen) >= 10
    tg = targets.copy()
    sel = np.union1d(rows, gen)
    tg[sel] = support_targets(logits[sel], w.vocab_real, w.temperature[sel], w.top_p[sel], w.top_k[sel], 3003)
    say("case: nucleus full size, groups 1")
    pol, ref, full = run_nucleus(logits, w.vocab_real, w.temperature, w.top_p, w.top_k, tg)
    check_ref_against_full(ref, full, logits, w.vocab_real, w.temperature, w.top_p, w.top_k, tg, TOL,
                           "nucleus full")
    assert np.isfinite(pol[sel]).all()
    _, n_alt = compare_rows(logits, w, tg, pol, ref, rows, "nucleus full, sampled rows")
    assert n_alt == 0
    compare_rows(logits, w, tg, pol, ref, gen, "nucleus full, rows with a zero or an outside token")


def test_per_request_sampled():
    """64 requests x 128 rows, T in {0.7, 1.0, 1.3}, top-p in {0.95, 0.99},
    top-k in {-1, 128}; two sampled rows per request, plus every row holding a
    zero or a token outside the window."""
    w = datagen.per_request()
    say("generating per-request workload")
    logits, targets = w.generate()
    rng = np.random.default_rng(4004)
    rows = np.array([r * 128 + int(rng.integers(0, 128)) for r in range(64)] +
                    [r * 128 + int(rng.integers(0, 128)) for r in range(64)])
    gen = general_path_rows(logits, w.vocab_real, zeros=True)
    report(f"per-request: {len(general_path_rows(logits, w.vocab_real))} general-path rows, "
           f"{len(gen)} rows with a zero or a token outside the window")
    assert len(gen) >= 10
    sel = np.union1d(rows, gen)
    tg = targets.copy()
    tg[sel] = support_targets(logits[sel], w.vocab_real, w.temperature[sel], w.top_p[sel], w.top_k[sel], 4005)
    for groups in (1, 4):
        say(f"case: per-request groups {groups}")
        pol, ref, full = run_nucleus(logits, w.vocab_real, w.temperature, w.top_p, w.top_k, tg, groups)
        check_ref_against_full(ref, full, logits, w.vocab_real, w.temperature, w.top_p, w.top_k, tg, TOL,
                               f"per-request g{groups}")
        compare_rows(logits, w, tg, pol, ref, np.unique(rows), f"per-request g{groups}, sampled rows")
        compare_rows(logits, w, tg, pol, ref, gen, f"per-request g{groups}, rows with a zero or an outside token")


def test_full_width_rows_with_and_without_a_search_at_every_grouping():
    """96 rows of 151936 real columns (the benchmark's value distribution) in
    one call, a third without a support search (top-p 1 and top-k off, or
    greedy), a third with top-p 0.95, a third with top-k 128 and top-p 0.99,
    at groups 1, 2, 4 and 8: with groups > 1 the float32 summaries of the rows
    without a search come from the grouped summary kernel and the searched rows
    are counted in one pass, so every grouping must give the same bytes, the
    rows without a search rlk_logp_full's reference bytes, and all rows the
    oracle's values."""
    vp, vr = datagen.QWEN3_VOCAB_PADDED, datagen.QWEN3_VOCAB_REAL
    n = 96
    rng = np.random.default_rng(4242)
    logits = np.full((n, vp), datagen.BF16_NEG_INF, dtype=np.uint16)
    for i in range(n):
        bits, _, _ = datagen.row_values((4242, i), vr, 2.5, 8.0 if i % 5 == 0 else None)
        logits[i, :vr] = bits
    kind = np.arange(n) % 3
    temps = np.where(kind == 0, np.where(np.arange(n) % 2 == 0, 0.7, 0.0), np.array([1.0, 0.7, 1.3])[np.arange(n) % 3])
    temps = temps.astype(np.float32)
    top_p = np.array([1.0, 0.95, 0.99], np.float32)[kind]
    top_k = np.array([-1, -1, 128], np.int32)[kind]
    tg = rng.integers(0, vr, size=n).astype(np.int64)
    say("case: full-width rows with and without a search, groups 1/2/4/8")
    check(logits, vr, temps, top_p, top_k, tg, "full width, mixed search")


def test_full_width_general_path_rows():
    """64 rows of 151936 real columns (benchmark's value distribution) with
    zeros, values below 2^-24 and, in some rows, a value below -4.24e9 injected:
    every row takes the general path (exact-maximum pass, 2048-bin histogram of
    counts and 64-bit masses, 32-key sub-passes, and its top-k branch), at
    top-k 128 or off, top-p 0.95 or 0.99, T 0.7 or 1.3."""
    vp, vr = datagen.QWEN3_VOCAB_PADDED, datagen.QWEN3_VOCAB_REAL
    n = 64
    rng = np.random.default_rng(8008)
    logits = np.full((n, vp), datagen.BF16_NEG_INF, dtype=np.uint16)
    for i in range(n):
        bits, _, _ = datagen.row_values((8008, i), vr, 2.5, 8.0 if i % 4 == 0 else None)
        cols = rng.choice(vr, 40, replace=False)
        bits[cols[:20]] = 0x0000
        bits[cols[20:30]] = 0x8000
        bits[cols[30:35]] = datagen.f32_to_bf16_bits(np.float32([1e-9]))[0]
        bits[cols[35:40]] = datagen.f32_to_bf16_bits(np.float32([-1e-9]))[0]
        if i % 8 == 3:
            bits[int(rng.integers(0, vr))] = datagen.f32_to_bf16_bits(np.float32([-5e9]))[0]
        logits[i, :vr] = bits
    assert len(general_path_rows(logits, vr)) == n
    temps = np.array([0.7, 1.3], np.float32)[np.arange(n) % 2]
    top_p = np.array([0.95, 0.99], np.float32)[(np.arange(n) // 2) % 2]
    top_k = np.array([-1, 128], np.int32)[(np.arange(n) // 4) % 2]
    tg = support_targets(logits, vr, temps, top_p, top_k, 8009)
    tg[::8] = rng.integers(0, vr, size=len(tg[::8]))     # some targets outside the support
    say("case: full-width general-path rows")
    check(logits, vr, temps, top_p, top_k, tg, "general path, full width", groups_list=(1, 8))


def test_every_window_class_as_a_top_k_boundary():
    """One row per class of the support window: each row holds every in-window
    BF16 value once (both zeros included, column order shuffled per row) and
    cuts top-k at a different class, so the support record's threshold must be
    exactly the k-th largest value, for every class of the window in turn. A
    sample of rows is compared with the oracle as well."""
    import torch
    mags = np.arange(0x3380, 0x4580, dtype=np.uint16)
    vals_bits = np.concatenate([mags, mags | np.uint16(0x8000), np.array([0x0000, 0x8000], np.uint16)])
    vals = datagen.bf16_bits_to_f32(vals_bits).astype(np.float64)
    order = np.argsort(-vals, kind="stable")
    sorted_vals = vals[order]
    n_tok = len(vals_bits)                       # 9218 tokens, 9217 classes
    vp = 9280                                    # multiple of 64
    ks = np.arange(1, n_tok + 1)                 # k = n_tok disables top-k (threshold -inf)
    n = len(ks)
    rng = np.random.default_rng(91)
    logits = np.full((n, vp), datagen.BF16_NEG_INF, dtype=np.uint16)
    for i in range(n):
        logits[i, :n_tok] = vals_bits[rng.permutation(n_tok)]
    temps = np.ones(n, np.float32)
    top_p = np.ones(n, np.float32)
    top_k = ks.astype(np.int32)
    am = np.argmax(datagen.bf16_bits_to_f32(logits[:, :n_tok]), axis=1).astype(np.int64)
    say(f"case: every window class as a top-k boundary ({n} rows x {vp})")
    lg = upload_logits(logits)
    for groups in (1, 4):
        pol, ref, lse, state = rlk.logp_nucleus(lg, upload(temps, torch.float32), upload(top_p, torch.float32),
                                                upload(top_k, torch.int32), upload(am, torch.int64),
                                                vocab_real=n_tok, groups=groups, return_state=True)
        torch.cuda.synchronize()
        _, thr, status = (to_host(a) for a in rlk.support_state_fields(state))
        want_thr = sorted_vals[ks - 1]
        want_thr = np.where(ks >= n_tok, -np.inf, want_thr)
        bad = np.flatnonzero(thr.astype(np.float64) != want_thr)
        assert bad.size == 0, f"groups {groups}: threshold wrong for k = {ks[bad[:5]]}: {thr[bad[:5]]} vs {want_thr[bad[:5]]}"
        assert np.all(status == 1)
        if groups == 1:
            first = to_host(pol).tobytes()
        else:
            assert to_host(pol).tobytes() == first
    sample = np.concatenate([np.arange(0, n, 97), [n - 1]])
    want_pol, _, infos = O.nucleus_logp(logits[sample], n_tok, temps[sample], top_p[sample], top_k[sample], am[sample])
    assert_nucleus_close(to_host(pol)[sample], want_pol, infos, what="window classes",
                         tol=row_tolerance(logits[sample], n_tok, temps[sample]))

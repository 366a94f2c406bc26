"""GPU parity of rlk_logp_backward (BF16 gradient of the reference and policy
logprobs with respect to the logits) and of the support record that
rlk_logp_nucleus emits for it, against the CPU oracle's float64 gradient.

Passages: RL-Kernel page "H100 canonical CP backward validation", Change
section (training back-propagates through the logprobs; the nonzero
gradients of the recorded runs came from the KL term); page "Configurable H100
consistency runs", mode/KL paragraph (reference over the full vocabulary,
policy over its top-p/top-k support).

Tolerance, per element (derived from the arithmetic, see grad_tolerance):
half a BF16 ulp of the result, plus the float32 error of the exponent
argument x*c - lse*log2(e) (relative 2^-21 times its magnitude plus a few
units), plus the error the backward inherits from its float32 inputs (the
forward's lse, lse_support, ref and policy values, measured against the
oracle row by row), plus a floor of 2^-125 |g|/T where exp2 may flush a
result below the float32 normal range. Outside it nothing is allowed:
NaN positions, zeros of zero/greedy rows and pad columns must match exactly.
"""
import numpy as np
import pytest

import datagen
import invariant_token_log_fp32_amd as rlk
from oracle import logp as O

from gpu_util import assert_close, exact_reference_rows, row_tolerance, say, to_host, upload, upload_logits

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


def bits_to_f64(bits):
    return datagen.bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def half_ulp_bf16(v):
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    e = np.where(a > 0, e, -125)
    return np.ldexp(1.0, np.maximum(e - 9, -134))


def dif(a, b):
    """|a - b|, 0 where both are the same (infinite) value."""
    return 0.0 if a == b else abs(a - b)


def grad_tolerance(bits_row, vp, vr, T, tg, g_r, g_p, lse_o, lse_g, ref_o, ref_g, pol_o=None, pol_g=None,
                   lse_s_o=None, lse_s_g=None, mask=None, want=None, got=None):
    x = bits_to_f64(bits_row[:vr])
    t = float(np.float32(T))
    z = O.scale_fp32(datagen.bf16_bits_to_f32(bits_row[:vr]), T)
    c = LOG2E / t
    with np.errstate(over="ignore", invalid="ignore"):
        p = np.exp(z - lse_o)
        kap_r = (np.abs(np.where(np.isfinite(x), x, 0.0)) * c + abs(lse_o) * LOG2E + 4.0) * 2.0 ** -21
        term = abs(g_r) / t * p * (kap_r + dif(lse_g, lse_o) * 1.01)
        if g_p:
            q = np.where(mask, np.exp(z - lse_s_o), 0.0)
            kap_p = (np.abs(np.where(np.isfinite(x), x, 0.0)) * c + abs(lse_s_o) * LOG2E + 4.0) * 2.0 ** -21
            term = term + abs(g_p) / t * q * (kap_p + dif(lse_s_g, lse_s_o) * 1.01)
    tol = np.zeros(vp)
    tol[:vr] = term
    # target column: (g_r * -expm1(ref) + g_p * -expm1(pol)) / T from the forward's float32 logprobs
    tt = abs(g_r) / t * (-np.expm1(ref_o) * 2.0 ** -20 + np.exp(min(ref_o, 0.0)) * dif(ref_g, ref_o) * 1.01)
    if g_p:
        tt += abs(g_p) / t * (-np.expm1(pol_o) * 2.0 ** -20 + np.exp(min(pol_o, 0.0)) * dif(pol_g, pol_o) * 1.01)
    tol[tg] = tt
    tol[:vr] += (abs(g_r) + abs(g_p)) / t * 2.0 ** -125
    big = np.maximum(np.abs(want), np.abs(got))
    return tol + half_ulp_bf16(big)


def compare_row(got_bits, want, tol, what):
    got = bits_to_f64(got_bits)
    nan_w = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan_w), f"{what}: NaN positions differ"
    fin = ~nan_w
    err = np.abs(got[fin] - want[fin])
    over = err - tol[fin]
    if over.max(initial=-1.0) > 0:
        j = int(np.flatnonzero(fin)[int(np.argmax(over))])
        raise AssertionError(f"{what}: column {j}: got {got[j]!r} want {want[j]!r} tol {tol[j]:.3e}")
    exact = datagen.f32_to_bf16_bits(want.astype(np.float32)) == np.asarray(got_bits, dtype=np.uint16)
    return int(exact[fin].sum()), int(fin.sum())


def run_forward(lg, t, p, k, tg, vr, vp=None, groups=1, host_logits=None):
    """GPU forward (nucleus with its support record). Its reference and lse
    equal rlk_logp_full's bytes on the rows that take the float32 shard sums,
    and lie within the tolerance of them on the rows that take the exact
    class masses."""
    import torch
    pol, ref, lse, state = rlk.logp_nucleus(lg, t, p, k, tg, vocab_real=vr, vocab_padded=vp, groups=groups,
                                            return_state=True)
    full, full_lse = rlk.logp_full(lg, t, tg, vocab_real=vr, vocab_padded=vp, groups=groups, return_lse=True)
    torch.cuda.synchronize()
    logits = host_logits if host_logits is not None else to_host(lg).view(np.uint16)
    exact = exact_reference_rows(logits, vr, to_host(t), to_host(p), to_host(k), to_host(tg))
    for a, b in ((ref, full), (lse, full_lse)):
        a, b = to_host(a), to_host(b)
        assert a[~exact].tobytes() == b[~exact].tobytes()
        assert_close(a[exact], b[exact], tol=row_tolerance(logits[exact], vr, to_host(t)[exact]), what="exact-mass reference")
    return pol, ref, lse, state


def check_batch(logits, vr, temps, top_p, top_k, targets, g_ref, g_pol, what, vp=None, out_pad=0, groups=1):
    """Forward + backward on the GPU; every row compared with the oracle."""
    import torch
    n = logits.shape[0]
    vp = vp or logits.shape[1]
    lg = upload_logits(logits)
    t = upload(temps, torch.float32)
    p = upload(top_p, torch.float32)
    k = upload(top_k, torch.int32)
    tg = upload(targets, torch.int64)
    pol, ref, lse, state = run_forward(lg, t, p, k, tg, vr, vp, groups)
    gr = upload(g_ref, torch.float32)
    gp = upload(g_pol, torch.float32)
    out = torch.full((n, vp + out_pad), 0x5A5A, dtype=torch.int16, device=lg.device)
    rlk.logp_backward(lg, t, tg, vocab_real=vr, vocab_padded=vp, ref_logp=ref, lse=lse, grad_ref=gr,
                      policy_logp=pol, support_state=state, grad_policy=gp, out=out)
    torch.cuda.synchronize()
    got = to_host(out).view(np.uint16)
    if out_pad:
        assert np.all(got[:, vp:] == 0x5A5A), f"{what}: columns beyond vocab_padded were written"
    lse_s_g, thr_g, status_g = (to_host(a) for a in rlk.support_state_fields(state))
    pol_g, ref_g, lse_g = to_host(pol), to_host(ref), to_host(lse)
    n_exact = n_all = n_amb = 0
    for i in range(n):
        T, tgi = float(temps[i]), int(targets[i])
        pi, ki = float(top_p[i]), int(top_k[i])
        pol_o, ref_o, info = O.nucleus_row(logits[i], vr, T, pi, ki, tgi, want_mask=True)
        _, lse_o = O.ref_logp_row(logits[i], vr, T, tgi)
        if info.ambiguous:  # the support may differ by one boundary class
            n_amb += 1
            continue
        want = O.grad_row(logits[i], vp, vr, T, tgi, float(g_ref[i]), float(g_pol[i]), pi, ki)
        row_what = f"{what} row {i} (T={T}, p={pi}, k={ki}, target {tgi})"
        if np.isnan(want).any() or T == 0 or not (g_ref[i] or g_pol[i]):
            # rows the rules settle: NaN on the real columns, or exact zeros
            got_f = bits_to_f64(got[i, :vp])
            assert np.array_equal(np.isnan(got_f), np.isnan(want)), f"{row_what}: NaN positions"
            fin = ~np.isnan(want)
            assert np.all(got_f[fin] == want[fin]), f"{row_what}: expected exact zeros"
            continue
        inside = info.support_mask is not None and bool(info.support_mask[tgi])
        g_p = float(g_pol[i]) if (inside and g_pol[i]) else 0.0
        if info.support_mask is not None:
            assert status_g[i] == (1 if inside else 0), f"{row_what}: support status"
            assert thr_g[i] == info.threshold, f"{row_what}: support threshold {thr_g[i]} vs {info.threshold}"
        tol = grad_tolerance(logits[i], vp, vr, T, tgi, float(g_ref[i]), g_p, lse_o, float(lse_g[i]), ref_o,
                             float(ref_g[i]), pol_o, float(pol_g[i]), info.lse_support, float(lse_s_g[i]),
                             info.support_mask, want, bits_to_f64(got[i, :vp]))
        e, a = compare_row(got[i, :vp], want, tol, row_what)
        n_exact += e
        n_all += a
    assert n_amb <= max(2, n // 50), f"{what}: {n_amb} ambiguous rows"
    if n_all:
        frac = n_exact / n_all
        say(f"{what}: {n_all} finite elements, {frac:.5f} equal to the rounded oracle value, {n_amb} ambiguous rows")
        assert frac > 0.98, f"{what}: only {frac:.4f} of the elements equal the rounded oracle value"
    return got


def test_tiny_reference_and_policy_terms():
    w = datagen.tiny()
    logits, targets = w.generate()
    rng = np.random.default_rng(41)
    cases = [(1.0, -1), (0.9, -1), (0.95, 50), (1.0, 10), (0.5, 3), (0.99, 128), (1.0, 1), (0.3, 1000)]
    rows, t, p, k, tg, gr, gp = [], [], [], [], [], [], []
    for ci, (pp, kk) in enumerate(cases):
        for i in range(w.n_rows):
            _, _, info = O.nucleus_row(logits[i], 1000, 1.0, pp, kk, 0, want_mask=True)
            inside = np.flatnonzero(info.support_mask)
            outside = np.flatnonzero(~info.support_mask)
            picks = list(rng.choice(inside, min(6, inside.size), replace=False))
            if outside.size:
                picks += list(rng.choice(outside, min(3, outside.size), replace=False))
            picks.append(int(targets[i]))
            for j, target in enumerate(picks):
                rows.append(logits[i])
                t.append([1.0, 0.7, 1.3][(ci + j) % 3])
                p.append(pp)
                k.append(kk)
                tg.append(int(target))
                gr.append([1.0, -0.37, 0.0, 2.5][j % 4])
                gp.append([0.8, 0.0, -1.9, 1.0][(j + ci) % 4])
    say(f"case: tiny, {len(rows)} rows over {len(cases)} support settings")
    check_batch(np.stack(rows), 1000, np.array(t, np.float32), np.array(p, np.float32), np.array(k, np.int32),
                np.array(tg, np.int64), np.array(gr, np.float32), np.array(gp, np.float32), "tiny", out_pad=8)


def test_ragged_shapes_and_groups():
    for seed, n, vp, vr, sigma, temp, pad in [(61, 9, 2048, 1999, 3.0, 0.7, 8), (62, 5, 4096, 700, 2.0, 0.8, 0),
                                              (63, 3, 512, 1, 2.0, 1.0, 24), (64, 6, 1024, 1021, 4.0, 1.3, 64)]:
        w = datagen.small(seed, n, vp, vr, sigma=sigma, temperature=temp)
        logits, targets = w.generate()
        rng = np.random.default_rng(seed)
        top_p = np.array([0.9, 1.0, 0.5, 0.99, 1.0, 0.7, 0.95, 1.0, 0.8][:n], np.float32)
        top_k = np.array([-1, 5, 50, -1, -1, 3, 100, 1, -1][:n], np.int32)
        gr = rng.normal(0, 1, n).astype(np.float32)
        gp = rng.normal(0, 1, n).astype(np.float32)
        for groups in (1, 4):
            say(f"case: ragged vocab {vp}/{vr}, groups {groups}")
            got = check_batch(logits, vr, w.temperature, top_p, top_k, targets, gr, gp, f"ragged {vp}/{vr} g{groups}",
                              out_pad=pad, groups=groups)
            if groups == 1:
                first = got.tobytes()
            assert got.tobytes() == first, "gradient bytes differ with groups"


def test_special_rows():
    """Zero upstream gradients, invalid rows, greedy rows, invalid top-p with
    and without a policy gradient, a target outside the support, a -inf
    target, -inf columns and a row holding a single finite value."""
    vp, vr = 1024, 1000
    rng = np.random.default_rng(9)
    base = rng.normal(0, 2.5, vr).astype(np.float32)
    rows, t, p, k, tg, gr, gp = [], [], [], [], [], [], []

    def add(vals, T, target, g_r, g_p, pp=1.0, kk=-1):
        r = np.full(vp, datagen.BF16_NEG_INF, dtype=np.uint16)
        r[:vr] = datagen.f32_to_bf16_bits(vals)
        rows.append(r); t.append(T); tg.append(target); gr.append(g_r); gp.append(g_p); p.append(pp); k.append(kk)

    add(base, float("nan"), 3, 0.0, 0.0)          # zero gradients: zeros even for an invalid row
    add(base, float("nan"), 3, 1.0, 0.0)          # invalid temperature
    add(base, 0.7, 1000, 1.0, 0.5)                # target out of range
    add(base, 0.7, -1, 0.0, 0.5, 0.9)             # negative target, policy term only
    nanrow = base.copy(); nanrow[17] = np.nan
    add(nanrow, 0.7, 3, 0.0, 1.0, 0.9)            # NaN logit, policy term only (status -2)
    add(base, 0.0, 3, 1.0, 1.0, 0.9, 5)           # greedy
    add(base, 0.7, 3, 1.0, 1.0, 1.5, -1)          # invalid top-p with a policy gradient: NaN
    add(base, 0.7, 3, 1.0, 0.0, 1.5, -1)          # invalid top-p, no policy gradient: reference term
    order = np.argsort(-base)
    add(base, 0.7, int(order[-1]), -0.5, 3.0, 0.5, 7)   # target outside the support
    neg = base.copy(); neg[::3] = -np.inf
    add(neg, 1.1, 0, 1.0, 1.0, 0.9)               # -inf target (column 0): d/dx_t = 1/T
    add(neg, 1.1, 1, 0.4, -0.6, 0.8, 20)          # -inf columns elsewhere
    one = np.full(vr, -np.inf, np.float32); one[500] = 3.0
    add(one, 0.9, 500, 1.0, 1.0, 0.5)             # a single finite value: gradient 0 everywhere
    add(base * 40, 0.7, int(order[0]), 1.0, 1.0, 0.9)   # large logits, target the argmax (p_t close to 1)
    logits = np.stack(rows)
    got = check_batch(logits, vr, np.array(t, np.float32), np.array(p, np.float32), np.array(k, np.int32),
                      np.array(tg, np.int64), np.array(gr, np.float32), np.array(gp, np.float32), "special rows")
    g = bits_to_f64(got)
    assert np.all(g[0] == 0) and np.all(np.isnan(g[1, :vr])) and np.all(g[1, vr:] == 0)
    assert np.all(g[5] == 0) and np.all(np.isnan(g[6, :vr])) and np.all(np.isfinite(g[7]))
    assert abs(g[9, 0] - 1 / 1.1) < 4e-3
    assert np.all(g[11, :500] == 0) and np.all(g[11, 501:] == 0)


def test_full_size_sampled_and_batch_invariant():
    """8192 x 152576 (real 151936) BF16 at T = 0.7 with top-p 0.95: sampled
    rows against the oracle; the gradient bytes of a row do not change with
    the batch it is computed in, and repeat calls are identical."""
    import torch
    w = datagen.nucleus()
    say("generating the 8192 x 152576 workload")
    logits, targets = w.generate()
    n, vp, vr = w.n_rows, w.vocab_padded, w.vocab_real
    rng = np.random.default_rng(12)
    gr = rng.normal(0, 1, n).astype(np.float32)
    gp = rng.normal(0, 1, n).astype(np.float32)
    lg = upload_logits(logits)
    t = upload(w.temperature, torch.float32)
    p = upload(w.top_p, torch.float32)
    k = upload(w.top_k, torch.int32)
    tg = upload(targets, torch.int64)
    say("case: full-size forward + backward")
    pol, ref, lse, state = run_forward(lg, t, p, k, tg, vr, host_logits=logits)
    kw = dict(vocab_real=vr, ref_logp=ref, lse=lse, grad_ref=upload(gr, torch.float32), policy_logp=pol,
              support_state=state, grad_policy=upload(gp, torch.float32))
    out = rlk.logp_backward(lg, t, tg, **kw)
    out2 = rlk.logp_backward(lg, t, tg, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "repeat calls differ"
    sub = np.sort(rng.choice(n, 37, replace=False))
    si = torch.as_tensor(sub, device=lg.device)
    sub_out = rlk.logp_backward(lg[si].contiguous(), t[si], tg[si], vocab_real=vr, ref_logp=ref[si], lse=lse[si],
                                grad_ref=kw["grad_ref"][si], policy_logp=pol[si], support_state=state[si].contiguous(),
                                grad_policy=kw["grad_policy"][si])
    torch.cuda.synchronize()
    assert torch.equal(sub_out.view(torch.int16), out[si].view(torch.int16)), "bytes depend on the batch"
    rows = sub[:10]
    got_rows = to_host(out[torch.as_tensor(rows, device=lg.device)].view(torch.int16))
    del out, out2, sub_out
    say(f"case: full-size oracle rows {list(rows)}")
    lse_s_g, thr_g, status_g = (to_host(a) for a in rlk.support_state_fields(state))
    pol_g, ref_g, lse_g = to_host(pol), to_host(ref), to_host(lse)
    n_exact = n_all = 0
    for j, i in enumerate(rows):
        T, tgi, pi, ki = float(w.temperature[i]), int(targets[i]), float(w.top_p[i]), int(w.top_k[i])
        pol_o, ref_o, info = O.nucleus_row(logits[i], vr, T, pi, ki, tgi, want_mask=True)
        if info.ambiguous:
            continue
        _, lse_o = O.ref_logp_row(logits[i], vr, T, tgi)
        want = O.grad_row(logits[i], vp, vr, T, tgi, float(gr[i]), float(gp[i]), pi, ki)
        inside = bool(info.support_mask[tgi])
        g_p = float(gp[i]) if inside else 0.0
        assert thr_g[i] == info.threshold and status_g[i] == (1 if inside else 0)
        bits = got_rows[j].view(np.uint16)
        tol = grad_tolerance(logits[i], vp, vr, T, tgi, float(gr[i]), g_p, lse_o, float(lse_g[i]), ref_o,
                             float(ref_g[i]), pol_o, float(pol_g[i]), info.lse_support, float(lse_s_g[i]),
                             info.support_mask, want, bits_to_f64(bits))
        e, a = compare_row(bits, want, tol, f"full row {i}")
        n_exact += e
        n_all += a
    say(f"full size: {n_exact / n_all:.5f} of {n_all} elements equal the rounded oracle value")
    assert n_exact / n_all > 0.98


def test_support_record_matches_oracle_and_groups():
    """rlk_support_state from every groups path: identical bytes, threshold
    and status equal to the oracle's, lse_support within the forward's
    tolerance, on the per-request mix of temperatures, top-p and top-k."""
    import torch
    w = datagen.per_request(rows_per_request=2)
    logits, targets = w.generate()
    lg = upload_logits(logits)
    args = (upload(w.temperature, torch.float32), upload(w.top_p, torch.float32), upload(w.top_k, torch.int32),
            upload(targets, torch.int64))
    first = None
    for groups in (1, 2, 4, 8):
        say(f"case: support record, groups {groups}")
        _, _, _, state = run_forward(lg, *args, w.vocab_real, groups=groups, host_logits=logits)
        b = to_host(state).tobytes()
        first = first or b
        assert b == first, f"support record bytes differ at groups {groups}"
    lse_s, thr, status = (to_host(a) for a in rlk.support_state_fields(state))
    tol = row_tolerance(logits, w.vocab_real, w.temperature)
    n_amb = 0
    for i in range(w.n_rows):
        pol_o, _, info = O.nucleus_row(logits[i], w.vocab_real, float(w.temperature[i]), float(w.top_p[i]),
                                       int(w.top_k[i]), int(targets[i]), want_mask=True)
        if info.ambiguous:
            n_amb += 1
            continue
        assert thr[i] == info.threshold, (i, thr[i], info.threshold)
        assert status[i] == (1 if info.support_mask[int(targets[i])] else 0)
        assert_close([lse_s[i]], [info.lse_support], tol=tol[i], what=f"lse_support row {i}")
    assert n_amb <= w.n_rows // 16, f"{n_amb} ambiguous rows"


def test_more_items_than_workgroups():
    """2^21 + 37 rows of a 64-column vocabulary (60 real): more (row, chunk)
    items than the backward launches workgroups, so workgroups take several
    items; the rows' bytes equal those of a small call on the same rows, and
    sampled rows match the oracle."""
    import torch
    n, vp, vr = (1 << 21) + 37, 64, 60
    w = datagen.small(71, n, vp, vr, sigma=2.0, temperature=0.9)
    say(f"case: {n} rows x {vp} columns")
    logits, targets = w.generate()
    lg = upload_logits(logits)
    t = upload(w.temperature, torch.float32)
    tg = upload(targets, torch.int64)
    gr = torch.linspace(-2, 2, n, device=lg.device, dtype=torch.float32)
    ref, lse = rlk.logp_full(lg, t, tg, vocab_real=vr, return_lse=True)
    out = rlk.logp_backward(lg, t, tg, vocab_real=vr, ref_logp=ref, lse=lse, grad_ref=gr)
    rows = torch.as_tensor(np.r_[0:40, n - 40:n], device=lg.device)
    small = rlk.logp_backward(lg[rows].contiguous(), t[rows], tg[rows], vocab_real=vr, ref_logp=ref[rows],
                              lse=lse[rows], grad_ref=gr[rows])
    torch.cuda.synchronize()
    assert torch.equal(small.view(torch.int16), out[rows].view(torch.int16))
    got = to_host(out[rows].view(torch.int16)).view(np.uint16)
    ref_h, lse_h, gr_h = to_host(ref[rows]), to_host(lse[rows]), to_host(gr[rows])
    for j, i in enumerate(to_host(rows)[::9]):
        jj = j * 9
        T, tgi = float(w.temperature[i]), int(targets[i])
        ref_o, lse_o = O.ref_logp_row(logits[i], vr, T, tgi)
        want = O.grad_row(logits[i], vp, vr, T, tgi, float(gr_h[jj]), 0.0)
        tol = grad_tolerance(logits[i], vp, vr, T, tgi, float(gr_h[jj]), 0.0, lse_o, float(lse_h[jj]), ref_o,
                             float(ref_h[jj]), want=want, got=bits_to_f64(got[jj]))
        compare_row(got[jj], want, tol, f"row {i}")

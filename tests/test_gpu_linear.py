"""GPU parity of the LM-head linear (rlk_linear) and the fused linear + logprob
(rlk_linear_logp) against the CPU oracle (oracle/linear.py).

Passages: RL-Kernel page "Reproduce and profile the Qwen3-8B TP4/CP2
experiment", section "Capture logs, status, and validation evidence" (the run
log is audited for the linear-logp backend); page "Configurable H100
consistency runs", sampling and mode/KL paragraphs.

Exactly summable inputs (small integers times powers of two, sparse
vocabulary rows) make every float32 partial sum exact in any order, so the
kernel's BF16 logits must equal the oracle's bit for bit, and the fused
logprob must match the oracle within the logprob tolerance (2e-5). With
random inputs the float32 accumulation order matters: a BF16 logit may then
differ from the oracle's correctly rounded one by one unit in the last place
(where the exact value lies within the accumulation error of a rounding
midpoint), and the fused logprob is compared with rlk_logp_full applied to
rlk_linear's logits (the same BF16 logits; only the order of the sum of
exponentials differs).
"""
import numpy as np
import pytest

import datagen
import invariant_token_log_fp32_amd as rlk
from oracle import linear as LIN

from gpu_util import assert_close, row_tolerance, say, to_host, upload, upload_logits

pytestmark = pytest.mark.gpu


def padded(bits, cols):
    """Device copy of a BF16 matrix with a row stride of ``cols`` (extra columns NaN)."""
    import torch
    n, d = bits.shape
    buf = np.full((n, cols), 0x7FC0, dtype=np.uint16)
    buf[:, :d] = bits
    t = torch.from_numpy(buf.view(np.int16)).to("cuda:0")
    return t[:, :d]


def run_linear(h, w, vp, out_cols=None):
    import torch
    n = h.shape[0]
    out = torch.full((n, out_cols or vp), 0x5A5A, dtype=torch.int16, device="cuda:0")
    rlk.linear(h, w, vocab_padded=vp, out=out)
    torch.cuda.synchronize()
    return to_host(out).view(np.uint16)


def params(n, vr, seed):
    rng = np.random.default_rng(seed)
    temps = rng.choice(np.array([0.7, 1.0, 1.3], np.float32), n)
    temps[::11] = 0.0
    tg = rng.integers(0, vr, n).astype(np.int64)
    return temps.astype(np.float32), tg


def test_exact_inputs_small_shapes():
    """Exactly summable inputs: the logits bit for bit, the logprob against the
    oracle. The last three shapes have more 256 x 256 tiles than a GPU has
    compute units, so a workgroup runs several tiles in a row, with one, two
    and three 64-deep stages per tile (the loads of a tile's first stages run
    during the previous tile's last ones; three stages flip the LDS buffer
    order from one tile to the next)."""
    import torch
    for seed, n, d, vr, vp, hpad, wpad, opad in [(1, 5, 64, 300, 320, 0, 8, 8), (2, 130, 128, 1000, 1024, 8, 0, 0),
                                                  (3, 257, 448, 1999, 2048, 16, 24, 64), (4, 1, 4096, 700, 768, 0, 0, 0),
                                                  (5, 129, 192, 64, 64, 0, 0, 0),
                                                  (6, 2000, 64, 10000, 10240, 0, 0, 0),
                                                  (7, 1500, 128, 12000, 12288, 8, 8, 0),
                                                  (8, 1100, 192, 14999, 15360, 0, 8, 8)]:
        say(f"case: exact {n} x {d} x {vr}/{vp}")
        hb, wb = datagen.linear_exact_inputs(seed, n, d, vr)
        h, w = padded(hb, d + hpad), padded(wb, d + wpad)
        got = run_linear(h, w, vp, vp + opad)
        want = LIN.logits_bf16(hb, wb, vp)
        assert np.array_equal(got[:, :vp], want), "logits differ from the exactly rounded oracle"
        if opad:
            assert np.all(got[:, vp:] == 0x5A5A), "columns beyond vocab_padded were written"
        temps, tg = params(n, vr, seed)
        tg_d = upload(tg, torch.int64)
        lp, lse = rlk.linear_logp(h, w, upload(temps, torch.float32), tg_d, vocab_padded=vp, return_lse=True)
        torch.cuda.synchronize()
        want_lp, want_lse = LIN.linear_logp(hb, wb, vp, temps, tg)
        tol = row_tolerance(want, vr, temps)
        assert_close(to_host(lp), want_lp, tol=tol, what=f"linear_logp {n}x{d}x{vr}")
        assert_close(to_host(lse), want_lse, tol=tol, what=f"lse {n}x{d}x{vr}")


def test_special_rows():
    """Greedy rows (ties across tiles, lowest column wins), invalid
    temperatures and targets, a target in the last (partial) tile."""
    import torch
    n, d, vr, vp = 12, 128, 1000, 1024
    hb, wb = datagen.linear_exact_inputs(9, n, d, vr)
    wb[[130, 700, 999]] = wb[5]               # the same logit in three tiles
    temps = np.array([0.0, 0.0, 0.0, 0.0, np.nan, -1.0, np.inf, 0.7, 0.7, 0.7, 1.3, 0.0], np.float32)
    tg = np.array([5, 130, 999, 6, 1, 1, 1, -1, 1000, 999, 998, 0], np.int64)
    lp = rlk.linear_logp(padded(hb, d), padded(wb, d), upload(temps, torch.float32), upload(tg, torch.int64),
                         vocab_padded=vp)
    torch.cuda.synchronize()
    want, _ = LIN.linear_logp(hb, wb, vp, temps, tg)
    assert_close(to_host(lp), want, what="special rows")


def test_special_logit_values():
    """Non-finite logits produced by the product itself: a NaN hidden value (a
    NaN row), +inf against a dense projection column (every logit +inf), one
    logit overflowing to +inf (2^100 * 2^100), -inf logits (one of them the
    target), plain rows, each at temperature 0.7, 1.3 and 0 (greedy); the
    summaries' NaN, +inf and -inf handling must give the oracle's values.
    The last rows hold a finite logit of 2^98, outside the scaled-logit domain
    |x * log2(e) / T| < 2^30: there the result must be the oracle's value or
    NaN, never another number."""
    import torch
    n, d, vr, vp = 18, 128, 1000, 1024
    say("case: special logits 18 x 128 x 1000")
    hb, wb = datagen.linear_exact_inputs(31, n, d, vr)
    big = datagen.f32_to_bf16_bits(np.array([2.0 ** 100, -(2.0 ** 100), np.inf, np.nan], np.float32))
    quarter = datagen.f32_to_bf16_bits(np.array([0.25], np.float32))[0]
    wb[:, 3] = quarter                 # a dense column: hidden value +inf there makes every logit +inf
    wb[:, 11] = 0
    wb[700, 11] = big[0]               # only column 700 sees hidden column 11
    wb[:, 12] = 0
    wb[[5, 6], 12] = big[0]            # columns 5 and 6 see hidden column 12
    hb[:, 11] = 0
    hb[:, 12] = 0
    kinds = []
    for r in range(n):
        kind = r // 3                  # 0 NaN row, 1 all +inf, 2 one +inf, 3 two -inf, 4 plain, 5 out of domain
        kinds.append(kind)
        if kind == 0:
            hb[r, 40] = big[3]
        elif kind == 1:
            hb[r, 3] = big[2]
        elif kind == 2:
            hb[r, 11] = big[0]
        elif kind == 3:
            hb[r, 12] = big[1]
        elif kind == 5:
            hb[r, 11] = quarter        # logit 700 = 2^98, finite
    temps = np.array([0.7, 1.3, 0.0] * 6, np.float32)
    tg = np.array([700 if k in (2, 5) else (5 if k == 3 else 17) for k in kinds], np.int64)
    tg[10] = 6                         # rows 9-11 hold two -inf logits (columns 5, 6); row 10 targets the other
    h, w = padded(hb, d), padded(wb, d)
    logits = run_linear(h, w, vp)
    want_logits = LIN.logits_bf16(hb, wb, vp)
    # a NaN logit may carry any sign and payload; every other logit is bit-exact
    gnan = (logits & 0x7FFF) > 0x7F80
    wnan = (want_logits & 0x7FFF) > 0x7F80
    assert np.array_equal(gnan, wnan), f"NaN logits differ: rows {np.flatnonzero((gnan != wnan).any(axis=1))}"
    diff = np.argwhere((logits != want_logits) & ~wnan)
    assert diff.size == 0, (f"logits differ from the exactly rounded oracle at {diff[:5].tolist()}: "
                            f"got {[hex(logits[tuple(i)]) for i in diff[:5]]} "
                            f"want {[hex(want_logits[tuple(i)]) for i in diff[:5]]}")
    t_d, tg_d = upload(temps, torch.float32), upload(tg, torch.int64)
    lp, lse = rlk.linear_logp(h, w, t_d, tg_d, vocab_padded=vp, return_lse=True)
    ref = rlk.logp_full(torch.from_numpy(logits.view(np.int16)).to("cuda:0"), t_d, tg_d, vocab_real=vr)
    torch.cuda.synchronize()
    lp, lse, ref = to_host(lp), to_host(lse), to_host(ref)
    want_lp, want_lse = LIN.linear_logp(hb, wb, vp, temps, tg)
    tol = row_tolerance(want_logits, vr, temps)
    inside = np.array([k != 5 for k in kinds])
    assert_close(lp[inside], want_lp[inside], tol=tol[inside], what="special logits: logp")
    assert_close(lse[inside], want_lse[inside], tol=tol[inside], what="special logits: lse")
    assert_close(lp[inside], ref[inside], tol=tol[inside], what="special logits: fused vs unfused")
    for r in np.flatnonzero(~inside):
        for name, got in (("fused", lp[r]), ("unfused", ref[r])):
            ok = np.isnan(got) or (np.isfinite(want_lp[r]) == np.isfinite(got) and
                                   (not np.isfinite(got) or abs(got - want_lp[r]) <= tol[r]))
            assert ok, f"row {r} (scaled logit beyond 2^30, {name}): {got} is neither NaN nor {want_lp[r]}"


def test_random_inputs_against_rlk_logp_full():
    import torch
    n, d, vr, vp = 300, 512, 5000, 5120
    say("case: random 300 x 512 x 5000")
    hb, wb = datagen.linear_inputs(21, n, d, vr)
    h, w = padded(hb, d), padded(wb, d)
    got = run_linear(h, w, vp)
    want = LIN.logits_bf16(hb, wb, vp)
    gx = datagen.bf16_bits_to_f32(got[:, :vr]).astype(np.float64)
    exact = LIN.acc_exact(hb, wb)
    wx = datagen.bf16_bits_to_f32(want[:, :vr]).astype(np.float64)
    # any float32 summation order of d products is within d * 2^-24 * sum|h w|
    # of the exact sum; one more rounding to BF16 adds half a unit of the result
    habs = np.abs(LIN.bf16_to_f64(hb))
    wabs = np.abs(LIN.bf16_to_f64(wb))
    bound = d * 2.0 ** -24 * (habs @ wabs.T) + np.abs(gx) * 2.0 ** -8 + 2.0 ** -133
    assert np.all(np.abs(gx - exact) <= bound), "a BF16 logit lies outside the float32 accumulation bound"
    frac = float(np.mean(gx != wx))
    say(f"random: {frac:.5f} of the logits differ from the correctly rounded value")
    assert frac < 0.05
    assert np.all(got[:, vr:] == 0xFF80)
    temps, tg = params(n, vr, 21)
    t_d, tg_d = upload(temps, torch.float32), upload(tg, torch.int64)
    lp, lse = rlk.linear_logp(h, w, t_d, tg_d, vocab_padded=vp, return_lse=True)
    lg = torch.from_numpy(got.view(np.int16)).to("cuda:0")
    ref, ref_lse = rlk.logp_full(lg, t_d, tg_d, vocab_real=vr, return_lse=True)
    torch.cuda.synchronize()
    assert_close(to_host(lp), to_host(ref), tol=row_tolerance(got, vr, temps), what="fused vs unfused logp")
    assert_close(to_host(lse), to_host(ref_lse), tol=row_tolerance(got, vr, temps), what="fused vs unfused lse")
    # batch invariance: the same rows in another batch give the same bytes
    sub = torch.as_tensor([299, 3, 150, 0, 77], device="cuda:0")
    lp2 = rlk.linear_logp(h[sub].contiguous(), w, t_d[sub], tg_d[sub], vocab_padded=vp)
    torch.cuda.synchronize()
    assert to_host(lp2).tobytes() == to_host(lp[sub]).tobytes()


def test_full_size_exact():
    """8192 x 4096 hidden states and a 151936 x 4096 projection (152576 padded
    columns), exactly summable: sampled rows of the logits bit for bit, the
    fused logprob against the oracle, and batch invariance."""
    import torch
    n, d, vr, vp = 8192, datagen.QWEN3_D_MODEL, datagen.QWEN3_VOCAB_REAL, datagen.QWEN3_VOCAB_PADDED
    say("generating exactly summable 8192 x 4096 and 151936 x 4096 inputs")
    hb, wb = datagen.linear_exact_inputs(31, n, d, vr)
    h = torch.from_numpy(hb.view(np.int16)).to("cuda:0")
    w = torch.from_numpy(wb.view(np.int16)).to("cuda:0")
    temps = np.full(n, 0.7, np.float32)
    temps[::97] = 0.0
    tg = np.random.default_rng(31).integers(0, vr, n).astype(np.int64)
    t_d, tg_d = upload(temps, torch.float32), upload(tg, torch.int64)
    say("case: full-size rlk_linear_logp")
    lp = rlk.linear_logp(h, w, t_d, tg_d, vocab_padded=vp)
    say("case: full-size rlk_linear")
    logits = rlk.linear(h, w, vocab_padded=vp)
    sub = torch.as_tensor([8191, 0, 4000, 97, 1234, 5555, 128, 127], device="cuda:0")
    lp_sub = rlk.linear_logp(h[sub].contiguous(), w, t_d[sub], tg_d[sub], vocab_padded=vp)
    torch.cuda.synchronize()
    assert to_host(lp_sub).tobytes() == to_host(lp[sub]).tobytes(), "bytes depend on the batch"
    rows = to_host(sub)
    got_rows = to_host(logits[sub].view(torch.int16)).view(np.uint16)
    want_rows = LIN.logits_bf16(hb[rows], wb, vp)
    assert np.array_equal(got_rows, want_rows)
    want_lp, _ = LIN.linear_logp(hb[rows], wb, vp, temps[rows], tg[rows])
    assert_close(to_host(lp)[rows], want_lp, tol=row_tolerance(want_rows, vr, temps[rows]), what="full size")
    # the fused path against rlk_logp_full on rlk_linear's logits, every row
    ref = rlk.logp_full(logits, t_d, tg_d, vocab_real=vr)
    torch.cuda.synchronize()
    assert_close(to_host(lp), to_host(ref), tol=2e-5, what="fused vs unfused, all rows")


def sharded_linear_logp(h, wb_host, t_d, tg_d, vr, vp, groups):
    """Each emulated rank gets only its own projection rows; summaries are
    concatenated in rank order and merged."""
    import torch
    n = h.shape[0]
    cols = vp // groups
    d = wb_host.shape[1]
    parts = []
    for r in range(groups):
        lo, hi = r * cols, min((r + 1) * cols, vr)
        rows = wb_host[lo:hi] if hi > lo else np.zeros((1, d), np.uint16)   # a valid pointer when the rank owns no row
        w_r = torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).to("cuda:0")
        parts.append(rlk.linear_logp_summaries(h, w_r, t_d, tg_d, rank=r, groups=groups, vocab_real=vr,
                                               vocab_padded=vp))
    return rlk.linear_logp_merge(torch.cat(parts), t_d, tg_d, n_rows=n, groups=groups, vocab_real=vr,
                                 vocab_padded=vp, return_lse=True)


def test_vocabulary_parallel_form_matches_one_gpu():
    """Ranks owning 1/2/4/8 of the columns (one rank owning no real row at
    8 ranks) give the bytes of the one-GPU call, greedy rows included."""
    import torch
    for seed, n, d, vr, vp in [(51, 300, 256, 3000, 4096), (52, 130, 128, 4096, 4096), (53, 17, 192, 999, 1024)]:
        hb, wb = datagen.linear_inputs(seed, n, d, vr)
        h = padded(hb, d)
        temps, tg = params(n, vr, seed)
        t_d, tg_d = upload(temps, torch.float32), upload(tg, torch.int64)
        one, one_lse = rlk.linear_logp(h, padded(wb, d), t_d, tg_d, vocab_padded=vp, return_lse=True)
        torch.cuda.synchronize()
        for groups in (1, 2, 4, 8):
            if (vp // groups) % 128:
                continue
            say(f"case: sharded linear-logp {n} x {d} x {vr}/{vp}, {groups} ranks")
            lp, lse = sharded_linear_logp(h, wb, t_d, tg_d, vr, vp, groups)
            torch.cuda.synchronize()
            assert to_host(lp).tobytes() == to_host(one).tobytes(), f"{groups} ranks: logp bytes differ"
            assert to_host(lse).tobytes() == to_host(one_lse).tobytes(), f"{groups} ranks: lse bytes differ"


def test_vocabulary_parallel_full_size_eight_ranks():
    import torch
    n, d, vr, vp = 8192, datagen.QWEN3_D_MODEL, datagen.QWEN3_VOCAB_REAL, datagen.QWEN3_VOCAB_PADDED
    say("case: sharded linear-logp at 8192 x 4096 x 151936, 8 ranks of 19072 columns")
    hb, wb = datagen.linear_inputs(61, n, d, vr)
    h = torch.from_numpy(hb.view(np.int16)).to("cuda:0")
    w = torch.from_numpy(wb.view(np.int16)).to("cuda:0")
    temps, tg = params(n, vr, 61)
    t_d, tg_d = upload(temps, torch.float32), upload(tg, torch.int64)
    one = rlk.linear_logp(h, w, t_d, tg_d, vocab_padded=vp)
    del w
    lp, _ = sharded_linear_logp(h, wb, t_d, tg_d, vr, vp, 8)
    torch.cuda.synchronize()
    assert to_host(lp).tobytes() == to_host(one).tobytes()

"""Helpers shared by the GPU tests: upload seeded inputs, call the C ABI through
the binding, and compare against the oracle with the tolerance the
specification fixes (2e-5 absolute for finite outputs; -inf and NaN
positions must agree exactly)."""
import sys

import numpy as np

TOL = 2e-5


# Lines that the test session prints in its terminal summary (counts that a
# passing run should still show: ambiguity-band rows, general-path rows).
REPORT = []


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def report(msg):
    say(msg)
    REPORT.append(msg)


def device():
    import torch
    return torch.device("cuda:0")


def upload_logits(arr: np.ndarray):
    import torch
    t = torch.from_numpy(arr.view(np.int16))
    return t.to(device(), non_blocking=False)


def upload(arr, dtype):
    import torch
    return torch.as_tensor(np.ascontiguousarray(arr), dtype=dtype, device=device())


def to_host(t):
    return t.detach().cpu().numpy()


def classify(v):
    v = np.asarray(v, dtype=np.float64)
    return np.where(np.isnan(v), 0, np.where(np.isposinf(v), 1, np.where(np.isneginf(v), 2, 3)))


def assert_close(got, want, tol=TOL, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    cg, cw = classify(got), classify(want)
    bad = np.flatnonzero(cg != cw)
    assert bad.size == 0, f"{what}: special-value mismatch at rows {bad[:10]}: got {got[bad[:10]]} want {want[bad[:10]]}"
    fin = cw == 3
    tol = np.broadcast_to(np.asarray(tol, dtype=np.float64), got.shape)
    if fin.any():
        err = np.abs(got[fin] - want[fin])
        over = err - tol[fin]
        worst = int(np.argmax(over))
        assert over.max() <= 0, (f"{what}: |err| {err[worst]:.3e} > tol {tol[fin][worst]:.1e} "
                                 f"(value {want[fin][worst]})")
        return float(err.max())
    return 0.0


# Rows whose scaled logits stay within this magnitude are compared at the flat
# 2e-5. Above it the error terms that grow with |x/T| (the relative rounding of
# c = fl32(log2(e)/T) in every exponent argument, and the float32 rounding of
# outputs whose magnitude reaches twice max|x/T|) are no longer small against
# the rest of the budget.
ORDINARY_MAX_Z = 64.0


def row_tolerance(logits, vocab_real, temps):
    """Per-row tolerance: 2e-5 absolute; for rows with max|x/T| above
    ORDINARY_MAX_Z, 2e-5 + 2^-22 * max|x/T| (one 2^-24 * max|z| for the rounding
    of c, one for the exponent argument's rounding near the row maximum, two
    for the float32 rounding of an output up to 2 * max|z| in magnitude)."""
    import datagen
    tol = np.full(logits.shape[0], TOL)
    for i in range(logits.shape[0]):
        x = datagen.bf16_bits_to_f32(logits[i, :vocab_real]).astype(np.float64)
        x = x[np.isfinite(x)]
        t = float(np.float32(temps[i]))
        if x.size and t > 0 and np.isfinite(t):
            zmax = float(np.abs(x).max()) / t
            if zmax > ORDINARY_MAX_Z:
                tol[i] += 2.0 ** -22 * zmax
    return tol


def assert_nucleus_close(pol_gpu, pol_want, infos, tol=TOL, what=""):
    """Policy comparison with the ambiguity band: a row whose top-p decision lies
    within the band may match the oracle under either neighbouring cut.

    Returns (rows the oracle flags as ambiguous, rows that matched only one of
    the flagged alternatives and not the oracle's own cut)."""
    pol_gpu = np.asarray(pol_gpu, dtype=np.float64)
    tol = np.broadcast_to(np.asarray(tol, dtype=np.float64), pol_gpu.shape)

    def same(c, g, t):
        if np.isnan(c) or np.isnan(g):
            return bool(np.isnan(c) and np.isnan(g))
        if np.isinf(c) or np.isinf(g):
            return c == g
        return abs(g - c) <= t

    n_amb = 0
    n_alt_only = 0
    for i, info in enumerate(infos):
        primary = same(pol_want[i], pol_gpu[i], tol[i])
        alt = info.ambiguous and any(same(c, pol_gpu[i], tol[i]) for c in info.alternatives)
        if info.ambiguous:
            n_amb += 1
        if alt and not primary:
            n_alt_only += 1
        assert primary or alt, (f"{what}: row {i}: got {pol_gpu[i]!r}, oracle {pol_want[i]!r}, "
                                f"alternatives {info.alternatives if info.ambiguous else []}")
    assert n_alt_only <= n_amb
    return n_amb, n_alt_only


# The nucleus entry point's window of BF16 classes: magnitudes [2^-24, 4096)
# of either sign, +-0, and -inf counted apart.
WINDOW_MAG_LO = 0x3380
WINDOW_N_MAG = 4608
SEARCH_ARG_LIMIT = 2.0 ** 20


def exact_reference_rows(logits, vocab_real, temps, top_p, top_k, targets):
    """Rows whose rlk_logp_nucleus reference comes from the exact integer class
    masses of the support search rather than from the float32 shard sums: rows
    that need a search (T > 0 finite, top-p in (0, 1], top-k -1 or 1..V, and
    top-p < 1 or top-k < V), whose real tokens all lie in the window or are
    -inf, with a target among the real columns, at least one finite token and
    |fl32(M * c)| < 2^20 for the row maximum M and c = fl32(log2(e) / T). The
    other rows' reference bytes equal rlk_logp_full's."""
    n = logits.shape[0]
    out = np.zeros(n, dtype=bool)
    log2e = np.float32(1.44269504088896340736)
    for lo in range(0, n, 256):
        hi = min(n, lo + 256)
        b = logits[lo:hi, :vocab_real]
        mag = b & 0x7FFF
        inw = ((mag >= WINDOW_MAG_LO) & (mag < WINDOW_MAG_LO + WINDOW_N_MAG)) | (mag == 0) | (b == 0xFF80)
        finite = b != 0xFF80
        for j, i in enumerate(range(lo, hi)):
            t = np.float32(temps[i])
            p = np.float32(top_p[i])
            k = int(top_k[i])
            tg = int(targets[i])
            if not (np.isfinite(t) and t > 0):
                continue
            if not (0 < p <= 1) or not (k == -1 or 1 <= k <= vocab_real):
                continue
            if not ((k != -1 and k < vocab_real) or p < 1):
                continue
            if not (0 <= tg < vocab_real) or not inw[j].all() or not finite[j].any():
                continue
            x = (b[j][finite[j]].astype(np.uint32) << 16).view(np.float32)
            c = np.float32(log2e / t)
            if abs(float(np.float32(x.max() * c))) < SEARCH_ARG_LIMIT:
                out[i] = True
    return out

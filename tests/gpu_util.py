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

"""Helpers shared by the GPU tests: upload seeded inputs, call the C ABI through
the binding, and compare against the oracle with the tolerance the
specification fixes (2e-5 absolute for finite outputs; -inf and NaN
positions must agree exactly)."""
import sys

import numpy as np

TOL = 2e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


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


def row_tolerance(logits, vocab_real, temps):
    """2e-5 absolute, widened by 2^-20 * max|z| for rows whose scaled logits are
    large: an fp32 exponent argument carries a relative rounding of about 2^-24
    of |x/T|, which exceeds 2e-5 only when |x/T| is above about 300."""
    import datagen
    tol = np.full(logits.shape[0], TOL)
    for i in range(logits.shape[0]):
        x = datagen.bf16_bits_to_f32(logits[i, :vocab_real]).astype(np.float64)
        x = x[np.isfinite(x)]
        t = float(temps[i])
        if x.size and t > 0 and np.isfinite(t):
            tol[i] += 2.0 ** -20 * float(np.abs(x).max()) / t
    return tol


def assert_nucleus_close(pol_gpu, pol_want, infos, tol=TOL, what=""):
    """Policy comparison with the ambiguity band: a row whose top-p decision lies
    within the band may match the oracle under either neighbouring cut."""
    pol_gpu = np.asarray(pol_gpu, dtype=np.float64)
    tol = np.broadcast_to(np.asarray(tol, dtype=np.float64), pol_gpu.shape)
    n_amb = 0
    for i, info in enumerate(infos):
        cands = [pol_want[i]] + list(info.alternatives if info.ambiguous else [])
        ok = False
        for c in cands:
            if np.isnan(c) and np.isnan(pol_gpu[i]):
                ok = True
            elif np.isinf(c) or np.isinf(pol_gpu[i]):
                ok = ok or (c == pol_gpu[i])
            elif abs(pol_gpu[i] - c) <= tol[i]:
                ok = True
        if info.ambiguous:
            n_amb += 1
        assert ok, f"{what}: row {i}: got {pol_gpu[i]!r}, oracle {pol_want[i]!r}, alternatives {info.alternatives}"
    return n_amb

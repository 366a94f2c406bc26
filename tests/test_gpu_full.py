"""GPU parity of rlk_logp_full (through the C ABI) against the CPU oracle.

Defining passages: RL-Kernel page "Configurable H100 consistency runs"
(sampling, topology and mode/KL paragraphs) and page "Reproduce and profile
the Qwen3-8B TP4/CP2 experiment", section "How non-default CUDA topology
reuses TP4/CP2" (canonical 8-shard summaries merged in vocabulary order).
"""
import json
import math
import os
import zlib

import numpy as np
import pytest

import datagen
import invariant_token_log_fp32_amd as rlk
from oracle import logp as O

from gpu_util import TOL, assert_close, row_tolerance, say, to_host, upload, upload_logits

pytestmark = pytest.mark.gpu

GROUPS = (1, 2, 4, 8)


def run_full(logits_np, vr, temps, targets, groups=1, vp=None, return_lse=True):
    import torch
    lg = upload_logits(logits_np)
    t = upload(temps, torch.float32)
    tg = upload(targets, torch.int64)
    out, lse = rlk.logp_full(lg, t, tg, vocab_real=vr, vocab_padded=vp, groups=groups, return_lse=True)
    torch.cuda.synchronize()
    return to_host(out), to_host(lse)


def oracle_full(logits_np, vr, temps, targets):
    return O.ref_logp(logits_np, vr, temps, targets)


def test_tiny_matches_golden_and_oracle_for_every_target():
    say("case: tiny, 4 rows x every target")
    w = datagen.tiny()
    logits, targets = w.generate()
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny.json")))
    for groups in GROUPS:
        got, lse = run_full(logits, 1000, w.temperature, targets, groups)
        for r in g["rows"]:
            assert abs(got[r["row"]] - r["ref_logp"]) <= TOL
            assert abs(lse[r["row"]] - r["lse"]) <= TOL
    # every real token of every row as a target (4000 rows, replicas of 4 rows)
    rep = np.repeat(logits, 1000, axis=0)
    tg = np.tile(np.arange(1000), 4)
    temps = np.ones(4000, dtype=np.float32)
    want, want_lse = oracle_full(rep, 1000, temps, tg)
    for groups in GROUPS:
        got, lse = run_full(rep, 1000, temps, tg, groups)
        assert_close(got, want, what=f"tiny all targets g{groups}")
        for i in range(4):
            blk = lse[i * 1000:(i + 1) * 1000]
            assert np.all(blk.view(np.uint32) == blk[0].view(np.uint32)), "lse differs between replicas of a row"
            assert abs(math.fsum(np.exp(got[i * 1000:(i + 1) * 1000].astype(np.float64))) - 1.0) < 3e-5


SHAPES = [
    # (name, n_rows, vocab_padded, vocab_real, row_stride, sigma, temperatures, spike)
    ("qwen-37rows-mixedT", 37, 152576, 151936, 152576, 2.5, [0.7, 1.0, 1.3, 0.5, 2.0, 0.25], 8.0),
    ("ragged-tail-1999", 9, 2048, 1999, 2048, 3.0, [1.0, 0.7], None),
    ("single-real-column", 3, 512, 1, 512, 2.0, [1.0], None),
    ("no-pads", 5, 512, 512, 512, 2.0, [0.9], None),
    ("padded-stride", 6, 1024, 1000, 1088, 3.0, [1.1], None),
    ("shards-partly-empty", 4, 4096, 700, 4096, 2.0, [0.8], None),
    ("wide-sigma", 5, 8192, 8000, 8192, 12.0, [1.0, 0.3], None),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_parity_small_shapes_all_groups(shape):
    name, n, vp, vr, stride, sigma, temps, spike = shape
    say(f"case: {name}")
    w = datagen.small(zlib.crc32(name.encode()) % 1000 + 31, n, vp, vr, sigma=sigma,
                      temperature=np.resize(np.array(temps, np.float32), n), spike=spike, row_stride=stride)
    logits, targets = w.generate()
    want, want_lse = oracle_full(logits, vr, w.temperature, targets)
    ref_bytes = None
    for groups in GROUPS:
        got, lse = run_full(logits, vr, w.temperature, targets, groups, vp=vp)
        tol = row_tolerance(logits, vr, w.temperature)
        assert_close(got, want, tol=tol, what=f"{name} g{groups}")
        assert_close(lse, want_lse, tol=tol, what=f"{name} lse g{groups}")
        if ref_bytes is None:
            ref_bytes = (got.tobytes(), lse.tobytes())
        assert (got.tobytes(), lse.tobytes()) == ref_bytes, f"{name}: bytes differ between groups"


@pytest.mark.parametrize("fill", ["nan", "posinf", "huge"])
def test_pad_columns_never_read(fill):
    say(f"case: poisoned pads {fill}")
    base = datagen.small(501, 6, 2048, 1999, sigma=3.0, temperature=0.7, row_stride=2048)
    poisoned = datagen.small(501, 6, 2048, 1999, sigma=3.0, temperature=0.7, row_stride=2048, pad=fill)
    a, ta = base.generate()
    b, tb = poisoned.generate()
    for groups in GROUPS:
        ga, la = run_full(a, 1999, base.temperature, ta, groups)
        gb, lb = run_full(b, 1999, poisoned.temperature, tb, groups)
        assert ga.tobytes() == gb.tobytes() and la.tobytes() == lb.tobytes()


def _bf16(v):
    return datagen.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def test_special_rows():
    """Greedy rows, invalid temperatures and targets, -inf / NaN / +inf logits,
    an all -inf row, and rows that take the exact two-pass recompute."""
    say("case: special rows")
    vp, vr = 4096, 4000
    rng = np.random.default_rng(7)
    rows, temps, tgs = [], [], []

    def add(row_vals, t, tg):
        r = np.full(vp, datagen.BF16_NEG_INF, dtype=np.uint16)
        r[:vr] = _bf16(row_vals)
        rows.append(r)
        temps.append(t)
        tgs.append(tg)

    base = rng.normal(0, 2.0, vr).astype(np.float32)
    tied = base.copy()
    tied[[100, 2500, 3999]] = 20.0
    for tg in (100, 2500, 3999, 5):
        add(tied, 0.0, tg)                   # greedy with ties: lowest index wins
    add(tied, -0.0, 100)                     # -0 is greedy too
    add(base, float("nan"), 3)               # invalid temperature
    add(base, -1.0, 3)
    add(base, float("inf"), 3)
    add(base, 0.7, -1)                       # invalid targets
    add(base, 0.7, vr)
    add(base, 0.7, vp - 1)                   # pad column is not a valid target
    neg = base.copy()
    neg[::3] = -np.inf
    add(neg, 0.7, 0)                         # target with -inf logit
    add(neg, 0.7, 1)
    add(np.full(vr, -np.inf, np.float32), 1.0, 0)   # all -inf: NaN
    nanrow = base.copy()
    nanrow[1234] = np.nan
    add(nanrow, 1.0, 0)
    infrow = base.copy()
    infrow[77] = np.inf
    add(infrow, 1.0, 0)
    far = np.full(vr, -100.0, np.float32)    # first chunks far below the maximum
    far[3900] = 100.0
    far[3000:3010] = 95.0
    add(far, 0.5, 3900)
    add(far, 0.5, 3005)
    lowrow = np.full(vr, -3000.0, np.float32)  # all very negative logits
    lowrow[10] = -2990.0
    add(lowrow, 1.0, 10)
    add(lowrow, 1.0, 11)
    add(base * 40.0, 0.05, int(np.argmax(base)))  # huge scaled range
    logits = np.stack(rows)
    temps = np.array(temps, dtype=np.float32)
    tgs = np.array(tgs, dtype=np.int64)
    want, want_lse = oracle_full(logits, vr, temps, tgs)
    ref = None
    for groups in GROUPS:
        got, lse = run_full(logits, vr, temps, tgs, groups)
        assert_close(got, want, tol=row_tolerance(logits, vr, temps), what=f"special g{groups}")
        if ref is None:
            ref = got.tobytes()
        assert got.tobytes() == ref


def test_empty_batch():
    import torch
    say("case: empty batch")
    lg = torch.zeros((0, 1024), dtype=torch.int16, device="cuda:0")
    t = torch.zeros(0, dtype=torch.float32, device="cuda:0")
    tg = torch.zeros(0, dtype=torch.int64, device="cuda:0")
    out = rlk.logp_full(lg, t, tg, vocab_real=1000, vocab_padded=1024)
    assert out.numel() == 0


@pytest.fixture(scope="module")
def full_workload():
    w = datagen.full()
    say("generating the 8192 x 152576 workload")
    logits, targets = w.generate()
    return w, logits, targets


def test_full_size_sampled_rows_and_groups(full_workload):
    """8192 x 152576 BF16 at T = 0.7 in the benchmark's launch configuration
    (groups = 1), sampled rows against the oracle; groups 2/4/8 byte-identical."""
    w, logits, targets = full_workload
    say("case: full size, groups 1")
    got, lse = run_full(logits, w.vocab_real, w.temperature, targets, 1)
    assert np.isfinite(got).all() and np.isfinite(lse).all()
    rows = np.random.default_rng(99).choice(w.n_rows, 48, replace=False)
    rows = np.concatenate([rows, [0, w.n_rows - 1]])
    want, want_lse = oracle_full(logits[rows], w.vocab_real, w.temperature[rows], targets[rows])
    assert_close(got[rows], want, what="full sampled")
    assert_close(lse[rows], want_lse, what="full sampled lse")
    for groups in (2, 4, 8):
        say(f"case: full size, groups {groups}")
        g2, l2 = run_full(logits, w.vocab_real, w.temperature, targets, groups)
        assert g2.tobytes() == got.tobytes() and l2.tobytes() == lse.tobytes()


def test_reference_exponent_recompute_paths():
    """Shards whose first chunk (2048 columns) lies far below later columns: the
    streaming reference then either holds large finite terms or overflows and
    takes the exact two-pass recompute. Both must match the oracle and be
    identical across groups."""
    say("case: recompute paths")
    vp, vr = 32768, 32000
    rng = np.random.default_rng(11)
    rows, temps, tgs = [], [], []
    for case in range(6):
        v = rng.normal(0, 1.0, vr).astype(np.float32)
        shard = vp // 8
        for s in range(8):
            lo = s * shard
            v[lo:lo + 2048] -= 60.0            # first chunk of every shard far below
        if case % 2 == 0:
            v[5 * shard + 3000] = 120.0        # overflow of 2^(x*c - r): recompute
        else:
            v[5 * shard + 3000] = 10.0         # large finite terms, no recompute
        r = np.full(vp, datagen.BF16_NEG_INF, dtype=np.uint16)
        r[:vr] = _bf16(v)
        rows.append(r)
        temps.append([0.5, 1.0, 0.7][case % 3])
        tgs.append([5 * shard + 3000, 17, 5 * shard + 3100][case % 3])
    logits = np.stack(rows)
    temps = np.array(temps, dtype=np.float32)
    tgs = np.array(tgs, dtype=np.int64)
    want, want_lse = oracle_full(logits, vr, temps, tgs)
    ref = None
    for groups in GROUPS:
        got, lse = run_full(logits, vr, temps, tgs, groups)
        tol = row_tolerance(logits, vr, temps)
        assert_close(got, want, tol=tol, what=f"recompute g{groups}")
        assert_close(lse, want_lse, tol=tol, what=f"recompute lse g{groups}")
        if ref is None:
            ref = got.tobytes()
        assert got.tobytes() == ref

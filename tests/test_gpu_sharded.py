"""GPU tests of the vocabulary-parallel form: rlk_logp_shard_summaries on each
rank's column slice, then rlk_logp_merge on the rank-ordered concatenation.

Passage: RL-Kernel page "Reproduce and profile the Qwen3-8B TP4/CP2
experiment", section "How non-default CUDA topology reuses TP4/CP2": logp
emits per-virtual-shard vocabulary summaries and merges them in fixed
global-vocabulary order, a coarser physical rank owning several virtual
shards; page "Configurable H100 consistency runs", topology paragraph: fixed
virtual TP8 partitions of the padded vocabulary. Each emulated rank sees only
its own slice buffer; the merged bytes must equal the one-GPU path's for every
number of ranks, and the values must match the oracle.
"""
import numpy as np
import pytest

import datagen
import invariant_token_log_fp32_amd as rlk
from oracle import logp as O

from gpu_util import assert_close, row_tolerance, say, to_host, upload, upload_logits

pytestmark = pytest.mark.gpu


def sharded(lg, temps, tg, vr, vp, groups, pad_cols=0):
    """Each rank's slice as its own buffer (optionally with a padded row stride)."""
    import torch
    n = lg.shape[0]
    cols = vp // groups
    parts = []
    for r in range(groups):
        buf = torch.full((n, cols + pad_cols), 0x7FC0, dtype=torch.int16, device=lg.device)  # NaN past the slice
        buf[:, :cols] = lg[:, r * cols:(r + 1) * cols]
        parts.append(rlk.logp_shard_summaries(buf, temps, tg, rank=r, groups=groups, vocab_real=vr, vocab_padded=vp))
    gathered = torch.cat(parts)
    return rlk.logp_merge(gathered, temps, tg, n_rows=n, groups=groups, vocab_real=vr, vocab_padded=vp,
                          return_lse=True)


def check_workload(logits, temps, targets, vr, vp, what, pad_cols=0):
    import torch
    lg = upload_logits(logits)
    t = upload(temps, torch.float32)
    tg = upload(targets, torch.int64)
    full, full_lse = rlk.logp_full(lg, t, tg, vocab_real=vr, vocab_padded=vp, return_lse=True)
    torch.cuda.synchronize()
    full_b, lse_b = to_host(full).tobytes(), to_host(full_lse).tobytes()
    for groups in (1, 2, 4, 8):
        say(f"case: {what}, {groups} ranks")
        got, lse = sharded(lg, t, tg, vr, vp, groups, pad_cols)
        torch.cuda.synchronize()
        assert to_host(got).tobytes() == full_b, f"{what}: merged bytes differ from the one-GPU path ({groups} ranks)"
        assert to_host(lse).tobytes() == lse_b
    return to_host(full)


def test_tiny_and_ragged_shapes():
    for seed, n, vp, vr, sigma, t, pad in [(1001, 4, 1024, 1000, 3.0, 1.0, 0), (61, 9, 2048, 1999, 3.0, 0.7, 8),
                                          (62, 5, 4096, 700, 2.0, 0.8, 0), (63, 3, 512, 1, 2.0, 1.0, 24)]:
        w = datagen.small(seed, n, vp, vr, sigma=sigma, temperature=t)
        logits, targets = w.generate()
        got = check_workload(logits, w.temperature, targets, vr, vp, f"vocab {vp}/{vr}", pad)
        want, _ = O.ref_logp(logits, vr, w.temperature, targets)
        assert_close(got, want, tol=row_tolerance(logits, vr, w.temperature), what=f"vocab {vp}/{vr}")


def test_special_rows_across_ranks():
    """Greedy ties in different ranks' slices, invalid temperatures and
    targets, -inf targets, and a target in the last rank's slice."""
    vp, vr = 4096, 4000
    rng = np.random.default_rng(5)
    base = rng.normal(0, 2.0, vr).astype(np.float32)
    rows, temps, tgs = [], [], []

    def add(vals, t, tg):
        r = np.full(vp, datagen.BF16_NEG_INF, dtype=np.uint16)
        r[:vr] = datagen.f32_to_bf16_bits(vals)
        rows.append(r)
        temps.append(t)
        tgs.append(tg)

    tied = base.copy()
    tied[[700, 2100, 3999]] = 30.0   # maxima in three different ranks at groups 4 and 8
    for tg in (700, 2100, 3999, 5):
        add(tied, 0.0, tg)
    neg = base.copy()
    neg[::5] = -np.inf
    add(neg, 0.7, 0)
    add(neg, 0.7, 3999)
    add(base, float("nan"), 1)
    add(base, 0.7, -1)
    add(base, 0.7, vr)
    add(base, 1.3, 3998)
    logits = np.stack(rows)
    temps = np.array(temps, np.float32)
    tgs = np.array(tgs, np.int64)
    got = check_workload(logits, temps, tgs, vr, vp, "special rows")
    want, _ = O.ref_logp(logits, vr, temps, tgs)
    assert_close(got, want, tol=row_tolerance(logits, vr, temps), what="special rows")


def test_full_size_eight_ranks():
    """8192 x 152576 BF16 split into 2, 4 and 8 rank slices (8 x 19072 columns
    at 8 ranks); merged bytes equal the one-GPU path; sampled rows vs oracle."""
    w = datagen.full()
    say("generating the 8192 x 152576 workload")
    logits, targets = w.generate()
    got = check_workload(logits, w.temperature, targets, w.vocab_real, w.vocab_padded, "full size")
    rows = np.random.default_rng(8).choice(w.n_rows, 24, replace=False)
    want, _ = O.ref_logp(logits[rows], w.vocab_real, w.temperature[rows], targets[rows])
    assert_close(got[rows], want, what="full size sampled")

"""Byte invariance of the outputs across batch composition, row order, shard
grouping and repeated runs (the pages' acceptance metric is zero byte
mismatches between training and rollout logprobs: page "H100 rollout context
parallelism", "Measured results"; page "H100 canonical CP backward
validation", title block).

Workload: 64 ragged sequences with lengths uniform in 1..1024 (about 32.8k
rows) of 152576-wide BF16 logits, T = 0.7, top-p 0.95, top-k off; evaluated as
batches of 1, 7 and 64 sequences, with the 8 shards grouped as 1/2/4/8
physical blocks, and under a seeded row permutation.
"""
import numpy as np
import pytest

import datagen
import invariant_token_log_fp32_amd as rlk
from oracle import logp as O

from gpu_util import assert_close, assert_nucleus_close, say, to_host, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def stress():
    import torch
    w = datagen.stress()
    say(f"generating stress workload: {w.n_rows} rows")
    dev = torch.device("cuda:0")
    logits_dev = torch.empty((w.n_rows, w.row_stride), dtype=torch.int16, device=dev)
    targets = np.empty(w.n_rows, dtype=np.int64)
    step = 2048
    for s in range(0, w.n_rows, step):
        rows = range(s, min(s + step, w.n_rows))
        block, tg = w.generate(rows=rows)
        targets[s:s + len(block)] = tg
        logits_dev[s:s + len(block)].copy_(torch.from_numpy(block.view(np.int16)))
    torch.cuda.synchronize()
    say("stress workload on device")
    params = dict(
        t=upload(w.temperature, torch.float32),
        p=upload(w.top_p, torch.float32),
        k=upload(w.top_k, torch.int32),
        tg=upload(targets, torch.int64),
    )
    return w, logits_dev, params, targets


def _eval(w, logits, prm, lo, hi, groups):
    """One call on rows [lo, hi) (a view: same stride, no copy)."""
    pol, ref = rlk.logp_nucleus(logits[lo:hi], prm["t"][lo:hi], prm["p"][lo:hi], prm["k"][lo:hi],
                                prm["tg"][lo:hi], vocab_real=w.vocab_real, vocab_padded=w.vocab_padded,
                                groups=groups)
    full, lse = rlk.logp_full(logits[lo:hi], prm["t"][lo:hi], prm["tg"][lo:hi], vocab_real=w.vocab_real,
                              vocab_padded=w.vocab_padded, groups=groups, return_lse=True)
    return pol, ref, full, lse


def _bytes(ts):
    import torch
    torch.cuda.synchronize()
    return [to_host(t).tobytes() for t in ts]


def test_batches_groups_permutation_and_repeat(stress):
    import torch
    w, logits, prm, targets = stress
    n = w.n_rows
    starts = np.concatenate([[0], np.cumsum(w.seq_lengths)])
    say("case: one call, groups 1")
    base = _bytes(_eval(w, logits, prm, 0, n, 1))
    mismatches = 0
    for groups in (1, 2, 4, 8):
        for bs in (1, 7, 64):
            say(f"case: batches of {bs} sequences, groups {groups}")
            outs = [torch.empty(n, dtype=torch.float32, device=logits.device) for _ in range(4)]
            for b in range(0, len(w.seq_lengths), bs):
                lo, hi = int(starts[b]), int(starts[min(b + bs, len(w.seq_lengths))])
                res = _eval(w, logits, prm, lo, hi, groups)
                for o, r in zip(outs, res):
                    o[lo:hi].copy_(r)
            got = _bytes(outs)
            for a, b in zip(got, base):
                mismatches += int(np.count_nonzero(np.frombuffer(a, np.uint32) != np.frombuffer(b, np.uint32)))
    assert mismatches == 0, f"{mismatches} byte-level mismatches across batches/groups"

    say("case: row permutation")
    perm = torch.from_numpy(np.random.default_rng(5005).permutation(n)).to(logits.device)
    lg_p = logits.index_select(0, perm)
    prm_p = {k: v.index_select(0, perm) for k, v in prm.items()}
    res = _eval(w, lg_p, prm_p, 0, n, 1)
    inv = torch.argsort(perm)
    got = _bytes([r.index_select(0, inv) for r in res])
    assert got == base, "outputs depend on row order"
    del lg_p

    say("case: repeat")
    assert _bytes(_eval(w, logits, prm, 0, n, 1)) == base

    say("case: oracle parity on sampled rows")
    rows = np.random.default_rng(77).choice(n, 16, replace=False)
    host = to_host(logits.index_select(0, torch.from_numpy(rows).to(logits.device))).view(np.uint16)
    pol = np.frombuffer(base[0], np.float32)[rows]
    ref = np.frombuffer(base[1], np.float32)[rows]
    want_pol, want_ref, infos = O.nucleus_logp(host, w.vocab_real, w.temperature[rows], w.top_p[rows],
                                               w.top_k[rows], targets[rows])
    assert_close(ref, want_ref, what="stress ref")
    assert_nucleus_close(pol, want_pol, infos, what="stress policy")

"""GPU test of rlk_logp_nucleus_noalloc (the entry point for callers that
cannot allocate): its outputs must equal rlk_logp_nucleus's byte for byte (the
same kernels; only where the shard summaries live differs), on two calls in a
row whose second input is smaller, at every grouping, including the largest
row count the static scratch holds."""
import numpy as np
import pytest

import datagen
import invariant_token_log_fp32_amd as rlk

from gpu_util import say, to_host, upload, upload_logits

pytestmark = pytest.mark.gpu


def _inputs(seed, n, vp, vr):
    w = datagen.small(seed, n, vp, vr, sigma=2.5, temperature=0.7)
    logits, targets = w.generate()
    rng = np.random.default_rng(seed)
    temps = rng.choice(np.array([0.7, 1.0, 1.3, 0.0], np.float32), n)
    top_p = rng.choice(np.array([0.95, 0.99, 1.0, 0.5], np.float32), n)
    top_k = rng.choice(np.array([-1, 128, 5, -1], np.int32), n)
    return logits, temps, top_p, top_k, targets


def _both(logits, temps, top_p, top_k, targets, vr, groups):
    import torch
    lg = upload_logits(logits)
    args = (lg, upload(temps, torch.float32), upload(top_p, torch.float32), upload(top_k, torch.int32),
            upload(targets, torch.int64))
    n = logits.shape[0]
    outs = {}
    for name in ("nucleus", "noalloc"):
        lse = torch.empty(n, dtype=torch.float32, device=lg.device)
        state = torch.empty((n, 4), dtype=torch.int32, device=lg.device)
        if name == "nucleus":
            pol, ref = rlk.logp_nucleus(*args, vocab_real=vr, groups=groups, lse_out=lse, state_out=state)
        else:
            pol, ref = rlk.logp_nucleus_noalloc(*args, vocab_real=vr, groups=groups, lse_out=lse, state_out=state)
        torch.cuda.synchronize()
        outs[name] = [to_host(t).tobytes() for t in (pol, ref, lse, state)]
    return outs


@pytest.mark.parametrize("groups", [1, 2, 4, 8])
def test_noalloc_matches_nucleus_on_two_calls(groups):
    vp, vr = 1024, 1000
    for step, n in enumerate((rlk.NOALLOC_MAX_ROWS, 777)):
        say(f"case: noalloc groups {groups}, call {step + 1}, {n} rows x {vp}")
        logits, temps, top_p, top_k, targets = _inputs(900 + 10 * groups + step, n, vp, vr)
        outs = _both(logits, temps, top_p, top_k, targets, vr, groups)
        for a, b, what in zip(outs["nucleus"], outs["noalloc"], ("policy", "reference", "lse", "state")):
            assert a == b, f"groups {groups}, call {step + 1}: {what} bytes differ"


def test_noalloc_full_width_rows_after_a_larger_call():
    """Benchmark-width rows (151936 real columns) after the calls above left
    other summaries in the scratch."""
    w = datagen.nucleus(n_rows=64)
    logits, targets = w.generate()
    for groups in (2, 8):
        say(f"case: noalloc full width, groups {groups}")
        outs = _both(logits, w.temperature, w.top_p, w.top_k, targets, w.vocab_real, groups)
        assert outs["nucleus"] == outs["noalloc"]


def test_noalloc_rejects_rows_beyond_the_scratch():
    import torch
    n = rlk.NOALLOC_MAX_ROWS + 1
    lg = torch.zeros((n, 64), dtype=torch.int16, device="cuda:0")
    with pytest.raises(rlk.RlkError) as e:
        rlk.logp_nucleus_noalloc(lg, 1.0, 0.9, -1, 0, vocab_real=64, groups=2)
    assert e.value.status == -7

"""CPU oracle for the LM-head linear layer and the fused linear + logprob.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module. The product path (the
HIP library and its Python binding) never imports, links or calls it, and this
module shares no code with that path; both take their inputs from ``datagen``.

Passages: RL-Kernel page "Reproduce and profile the Qwen3-8B TP4/CP2
experiment", section "Capture logs, status, and validation evidence" (the run
log is audited for the `linear-logp` backend: the LM-head linear fused with
the logprob); page "Configurable H100 consistency runs", sampling and mode/KL
paragraphs (BF16 model logits scaled by a float32 temperature; reference
logprob over the full real vocabulary).

What it computes, for hidden states h (n_rows x d_model) and the vocabulary
projection w (vocab_real x d_model), both BF16:

1. acc_ij = sum_k h_ik * w_jk in float64. Every product of two BF16 values
   is exact in float64 (8 + 8 significant bits); for the exactly summable
   inputs the tests use (small integers times powers of two) every partial
   sum is exact as well, and in general the float64 sum is within a few
   units of 2^-53 relative of the real value.
2. x_ij = bf16(acc_ij): acc rounded once, to nearest even, to 8 significant
   bits (the model's BF16 logits); overflow gives +-inf.
3. The logprob of the target under the temperature-scaled softmax of row i
   of x over the real vocabulary: ``oracle.logp.ref_logp`` on those logits
   (pads -inf), i.e. the plain definition in float64.
"""
from __future__ import annotations

import numpy as np

from . import logp as _logp

BF16_NEG_INF = 0xFF80


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def acc_exact(hidden_bits, weight_bits, chunk: int = 8192) -> np.ndarray:
    """float64 [n_rows, vocab_real] sums of products (item 1); the vocabulary
    rows are converted ``chunk`` at a time to bound memory."""
    h = bf16_to_f64(hidden_bits)
    wb = np.asarray(weight_bits)
    out = np.empty((h.shape[0], wb.shape[0]), dtype=np.float64)
    for lo in range(0, wb.shape[0], chunk):
        out[:, lo:lo + chunk] = h @ bf16_to_f64(wb[lo:lo + chunk]).T
    return out


def round_bf16(v) -> np.ndarray:
    """float64 -> BF16 bit patterns, one rounding to nearest even (item 2)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    flat = v.ravel()
    res = out.ravel()
    m, e = np.frexp(np.abs(flat))          # |v| = m * 2^e, m in [0.5, 1)
    # the quantum of an 8-bit significand is 2^(e - 8), but never below the
    # smallest BF16 subnormal 2^-133
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.round(np.ldexp(np.abs(flat), -q)), q)  # np.round: half to even
    r = np.where(np.isfinite(flat), r, np.abs(flat))
    r = np.copysign(r, flat)
    with np.errstate(over="ignore"):
        f32 = r.astype(np.float32)          # exact: r has at most 8 significant bits
    # values that round beyond the largest BF16 (0x7F7F = 3.3895e38) become inf
    big = np.abs(r) > float(np.frombuffer(np.array([0x7F7F0000], np.uint32).tobytes(), np.float32)[0])
    f32 = np.where(big, np.copysign(np.float32(np.inf), f32), f32)
    res[:] = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(flat)
    res[nan] = 0x7FC0
    return out


def logits_bf16(hidden_bits, weight_bits, vocab_padded: int) -> np.ndarray:
    """BF16 logits [n_rows, vocab_padded], pad columns -inf."""
    x = round_bf16(acc_exact(hidden_bits, weight_bits))
    n, vr = x.shape
    out = np.full((n, vocab_padded), BF16_NEG_INF, dtype=np.uint16)
    out[:, :vr] = x
    return out


def linear_logp(hidden_bits, weight_bits, vocab_padded: int, temperature, target):
    """(ref logprob, lse) per row (item 3)."""
    lg = logits_bf16(hidden_bits, weight_bits, vocab_padded)
    return _logp.ref_logp(lg, np.asarray(weight_bits).shape[0], temperature, target)

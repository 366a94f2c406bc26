"""CPU oracle for strict token log-probabilities (float64, numpy).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module. The product path (the
HIP library and its Python binding) never imports, links or calls it, and this
module shares no code with that path; both take their inputs from ``datagen``.

What it computes, per row i of BF16 logits ``x[i, j]`` (j < vocab_real):

1. Decode: ``x_j`` is the float32 value of the BF16 bits (exact widening).
   Columns at or beyond the real vocabulary are ignored whatever they hold
   (page "Configurable H100 consistency runs": support is computed from the
   real vocabulary; padded vocabulary 152576 in the topology paragraph).
2. Temperature: ``z_j = fl32(x_j / T)``, one IEEE float32 division rounded to
   nearest (same page, sampling paragraph: float32 temperature scaling after
   the BF16 logits). ``T == 0`` selects greedy sampling.
3. Reference logprob (same page, mode/KL paragraph: the KL reference is
   temperature-scaled over the full vocabulary):
   ``ref = z_t - log(sum_j exp(z_j))``, evaluated as
   ``M + log(fsum(exp(z_j - M)))`` with ``M = max z`` in float64.
   The per-shard (max, sum-exp) summaries merged in global vocabulary order
   on page "Reproduce and profile the Qwen3-8B TP4/CP2 experiment" (section
   "How non-default CUDA topology reuses TP4/CP2") are a regrouping of this
   same sum, so the oracle uses the plain definition.
4. Policy logprob (mode/KL paragraph: the policy logprob keeps its actual
   top-p/top-k sampling support; commands section: top-k is independent of
   top-p and temperature): distinct values of z in decreasing order form
   classes with counts c_r and masses w_r = c_r * exp(v_r - M).
   top-k (k != -1 and k < vocab_real) keeps the classes up to the first one
   whose cumulative count reaches k; top-p (p < 1) then keeps, among those,
   the classes up to the first one whose cumulative mass reaches p times
   their total. Every token tied with a boundary value is kept.
   ``pol = z_t - (M + log(sum of kept masses))`` if t is kept, else -inf; when
   the kept set is the whole real vocabulary, ``pol`` is ``ref`` itself.
5. Greedy (T == 0): a point mass on the lowest-index argmax of x; both
   outputs are 0 for that token and -inf for every other one.

6. Gradient (the training side consumes logprob gradients; page "H100
   canonical CP backward validation", "Change"): for upstream gradients
   g_ref, g_pol of one row,
   d/dx_j = (1/T) * ( [j == t] * (g_ref + g_pol') - g_ref * p_j
                      - g_pol' * [j in S] * q_j )
   with p = softmax(z) over the real vocabulary, q the softmax restricted to
   the support S, and g_pol' = g_pol when t is in S, else 0 (the policy
   logprob is the constant -inf there). The support is piecewise constant in
   x, so its boundaries carry no gradient. Pad columns get 0; a row with
   g_ref = g_pol = 0 or T = 0 (greedy: piecewise-constant logprob) gets 0; any
   other row whose forward is NaN gets NaN on its real columns.

Rows with an invalid temperature (NaN, +-inf, negative) or target (outside
[0, vocab_real)), or whose real logits contain NaN or +inf, or are all -inf,
give NaN for both outputs. An invalid top-p (outside (0, 1]) or top-k
(not -1 and not in [1, vocab_real]) gives NaN for the policy output only.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

NAN = float("nan")
NEG_INF = float("-inf")


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float32 values (the bits are the high half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def scale_fp32(x: np.ndarray, temperature: float) -> np.ndarray:
    """fl32(x / T) for every element, returned as float64 (exact widening)."""
    q = np.asarray(x, dtype=np.float32) / np.float32(temperature)
    return q.astype(np.float64)


def _t_valid(t: float) -> bool:
    return math.isfinite(t) and t >= 0.0


def _row_prelude(bits_row, vocab_real, temperature, target):
    """Shared validity checks; returns (x float32 real values, error or None)."""
    x = decode_bf16(np.asarray(bits_row)[:vocab_real])
    t = float(np.float32(temperature))
    if not _t_valid(t):
        return x, "temperature"
    if not (0 <= int(target) < vocab_real):
        return x, "target"
    if np.isnan(x).any() or np.isposinf(x).any():
        return x, "logits"
    if np.isneginf(x).all():
        return x, "empty"
    return x, None


def _greedy_index(x: np.ndarray) -> int:
    """Lowest index whose value equals the maximum (-0 and +0 compare equal)."""
    m = x.max()
    return int(np.flatnonzero(x == m)[0])


def ref_logp_row(bits_row, vocab_real: int, temperature: float, target: int) -> Tuple[float, float]:
    """Reference (full-vocabulary) logprob of ``target`` and the row's log-sum-exp.

    Returns (ref, lse); lse is NaN for greedy rows (no softmax is taken there).
    """
    x, err = _row_prelude(bits_row, vocab_real, temperature, target)
    if err is not None:
        return NAN, NAN
    t = float(np.float32(temperature))
    if t == 0.0:
        return (0.0 if _greedy_index(x) == int(target) else NEG_INF), NAN
    z = scale_fp32(x, t)
    m = float(z.max())
    s = math.fsum(np.exp(z - m).tolist())
    lse = m + math.log(s)
    return float(z[int(target)]) - lse, lse


@dataclass
class NucleusInfo:
    """Details of one row's support decision, for tests."""

    n_classes: int = 0
    r_k: int = -1          # last kept class after top-k (index into descending classes)
    r_p: int = -1          # last kept class after top-p
    r_star: int = -1       # last kept class overall
    support_size: int = 0
    frac_before: float = NAN   # cumulative top-p fraction before the boundary class
    frac_at: float = NAN       # cumulative top-p fraction including it
    alternatives: List[float] = field(default_factory=list)  # pol for neighbouring top-p cuts
    ambiguous: bool = False
    support_mask: Optional[np.ndarray] = None
    lse_support: float = NAN   # log of the support's sum of exp(z_j)
    threshold: float = NAN     # smallest kept BF16 logit value; -inf when the support is the whole real vocabulary


def _classes(z: np.ndarray):
    """Distinct values of z in decreasing order, their counts and the inverse map."""
    vals, inv, counts = np.unique(z, return_inverse=True, return_counts=True)
    vals = vals[::-1]
    counts = counts[::-1]
    inv = (len(vals) - 1) - inv
    return vals, counts, inv


def nucleus_row(bits_row, vocab_real: int, temperature: float, top_p: float, top_k: int,
                target: int, band: float = 2e-6, want_mask: bool = False):
    """Policy logprob over the top-k-then-top-p support, plus the reference logprob.

    Returns (pol, ref, NucleusInfo). ``band`` marks rows whose top-p decision
    lies within ``band`` of p on either side of the boundary class; for those,
    ``info.alternatives`` holds the policy value under each neighbouring cut.
    """
    info = NucleusInfo()
    ref, _ = ref_logp_row(bits_row, vocab_real, temperature, target)
    x, err = _row_prelude(bits_row, vocab_real, temperature, target)
    if err is not None:
        return NAN, NAN, info
    p = float(np.float32(top_p))
    k = int(top_k)
    if not (0.0 < p <= 1.0) or not (k == -1 or 1 <= k <= vocab_real):
        return NAN, ref, info
    t = float(np.float32(temperature))
    if t == 0.0:
        return ref, ref, info
    z = scale_fp32(x, t)
    m = float(z.max())
    vals, counts, inv = _classes(z)
    w = counts.astype(np.float64) * np.exp(vals - m)
    info.n_classes = len(vals)
    last = len(vals) - 1

    r_k = last
    if k != -1 and k < vocab_real:
        r_k = int(np.searchsorted(np.cumsum(counts), k, side="left"))
    info.r_k = r_k

    r_p = r_k
    if p < 1.0:
        zk = math.fsum(w[: r_k + 1].tolist())
        cum = np.cumsum(w[: r_k + 1])
        r_p = int(np.searchsorted(cum, p * zk, side="left"))
        r_p = min(r_p, r_k)
        info.frac_before = float(cum[r_p - 1] / zk) if r_p > 0 else 0.0
        info.frac_at = float(cum[r_p] / zk)
    info.r_p = r_p
    r_star = min(r_k, r_p)
    info.r_star = r_star
    info.support_size = int(counts[: r_star + 1].sum())
    if want_mask:
        info.support_mask = inv <= r_star
    info.lse_support = m + math.log(math.fsum(w[: r_star + 1].tolist()))
    info.threshold = NEG_INF if r_star == last else float(x[inv <= r_star].min())

    def pol_for(r_cut: int) -> float:
        if r_cut == last:
            return ref
        if inv[int(target)] > r_cut:
            return NEG_INF
        zs = math.fsum(w[: r_cut + 1].tolist())
        return float(z[int(target)]) - (m + math.log(zs))

    pol = pol_for(r_star)
    if p < 1.0:
        if r_p > 0 and info.frac_before >= p - band:
            info.ambiguous = True
            info.alternatives.append(pol_for(r_p - 1))
        if r_p < r_k and info.frac_at <= p + band:
            info.ambiguous = True
            info.alternatives.append(pol_for(r_p + 1))
    return pol, ref, info


# ---- batch helpers ---------------------------------------------------------

def ref_logp(logits: np.ndarray, vocab_real: int, temperature, target) -> Tuple[np.ndarray, np.ndarray]:
    """Row-by-row reference logprobs and log-sum-exps for a batch."""
    n = logits.shape[0]
    temperature = np.broadcast_to(np.asarray(temperature, dtype=np.float32), (n,))
    target = np.asarray(target, dtype=np.int64)
    ref = np.empty(n)
    lse = np.empty(n)
    for i in range(n):
        ref[i], lse[i] = ref_logp_row(logits[i], vocab_real, float(temperature[i]), int(target[i]))
    return ref, lse


def nucleus_logp(logits: np.ndarray, vocab_real: int, temperature, top_p, top_k, target, band=2e-6):
    """Row-by-row (policy, reference, infos) for a batch."""
    n = logits.shape[0]
    temperature = np.broadcast_to(np.asarray(temperature, dtype=np.float32), (n,))
    top_p = np.broadcast_to(np.asarray(top_p, dtype=np.float32), (n,))
    top_k = np.broadcast_to(np.asarray(top_k, dtype=np.int64), (n,))
    target = np.asarray(target, dtype=np.int64)
    pol = np.empty(n)
    ref = np.empty(n)
    infos = []
    for i in range(n):
        pol[i], ref[i], info = nucleus_row(logits[i], vocab_real, float(temperature[i]),
                                           float(top_p[i]), int(top_k[i]), int(target[i]), band)
        infos.append(info)
    return pol, ref, infos


def grad_row(bits_row, vocab_padded: int, vocab_real: int, temperature: float, target: int,
             g_ref: float, g_pol: float = 0.0, top_p: float = 1.0, top_k: int = -1) -> np.ndarray:
    """float64 gradient of g_ref * ref + g_pol * policy with respect to the row's
    logits (columns [0, vocab_padded)); see item 6 of the module docstring."""
    g = np.zeros(vocab_padded)
    g_ref = float(g_ref)
    g_pol = float(g_pol)
    if g_ref == 0.0 and g_pol == 0.0:
        return g
    x, err = _row_prelude(bits_row, vocab_real, temperature, target)
    if err is not None:
        g[:vocab_real] = NAN
        return g
    t = float(np.float32(temperature))
    if t == 0.0:
        return g
    z = scale_fp32(x, t)
    m = float(z.max())
    e = np.exp(z - m)
    zsum = math.fsum(e.tolist())
    p = e / zsum
    pol, _, info = nucleus_row(bits_row, vocab_real, temperature, top_p, top_k, target, want_mask=True)
    if g_pol != 0.0 and math.isnan(pol):
        g[:vocab_real] = NAN
        return g
    mask = info.support_mask
    gp = g_pol if (g_pol != 0.0 and mask[int(target)]) else 0.0
    out = -g_ref * p
    if gp != 0.0:
        es = np.where(mask, e, 0.0)
        q = es / math.fsum(es.tolist())
        out = out - gp * q
    out[int(target)] += g_ref + gp
    g[:vocab_real] = out / t
    return g

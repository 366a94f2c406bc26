"""CPU oracle for the deterministic FP32 gradient L2 norm (float64 / exact integers).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module. The product path (the
HIP library and its Python binding) never imports, links or calls it, and this
module shares no code with that path; both take their inputs from ``datagen``.

Passage: RL-Kernel page "H100 canonical CP backward validation", Change
section: Megatron's L2 norm sums the FP32 squares of the gradients in integer
exponent bins before the distributed reduction, so the norm that drives
gradient clipping does not depend on the order of the summation; Timing and
scope section: a 10M-element BF16-derived FP32 norm microbenchmark.

What it computes for a set of float32 values x_i (one or several tensors):

1. Squares: s_i = fl32(x_i * x_i), one IEEE float32 multiplication rounded to
   nearest even (the pages square in FP32). For BF16-derived values the
   square is exact (8 significant bits squared fit in 24).
2. Exponent bins (the integer encoding that travels through the reduction):
   for every biased exponent e of s_i in 0..254, bin[e] = sum of the 24-bit
   integer significands m_i (hidden bit included for e >= 1), so that
   s_i = m_i * 2^(max(e, 1) - 150) exactly. A square that is NaN counts in
   n_nan, one that is +inf (overflow or infinite x) in n_inf. This is the
   canonical spread of the words; any words with the same value
   sum_e bin[e] * 2^(max(e, 1) - 150) encode the same sum.
3. Sum of squares: the exact sum S of the s_i, rounded once to float64 (round
   to nearest even); NaN if any square is NaN, else +inf if any is +inf.
4. Norm: fl32(sqrt(fl64(S))) with IEEE square roots.

The plain definition of 3 is the exactly rounded sum of the squares, which is
``math.fsum`` of the float64 values of s_i; ``sumsq`` uses it. ``bins`` and
``sumsq_from_bins`` spell out the integer encoding of 2 and its exact value.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Iterable, List, Tuple

import numpy as np

N_BINS = 256  # biased exponents 0..254 hold values; 255 is never a finite square


def squares(x) -> np.ndarray:
    """fl32(x * x) element by element (IEEE float32 multiply)."""
    a = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        return a * a


def bins(xs: Iterable) -> Tuple[List[int], int, int]:
    """(bin[0..255], n_nan, n_inf) over every array in ``xs`` (item 2)."""
    out = [0] * N_BINS
    n_nan = n_inf = 0
    for x in xs:
        s = squares(x).ravel()
        u = s.view(np.uint32).astype(np.uint64)
        e = (u >> np.uint64(23)) & np.uint64(0xFF)
        frac = u & np.uint64(0x7FFFFF)
        special = e == 255
        n_nan += int(np.count_nonzero(special & (frac != 0)))
        n_inf += int(np.count_nonzero(special & (frac == 0)))
        m = np.where(e > 0, frac | np.uint64(0x800000), frac)
        fin = ~special
        # per-exponent integer sums; np.add.at on uint64 is exact (each
        # significand < 2^24, fewer than 2^40 terms)
        acc = np.zeros(N_BINS, dtype=np.uint64)
        np.add.at(acc, e[fin].astype(np.int64), m[fin])
        for k in range(N_BINS):
            out[k] += int(acc[k])
    return out, n_nan, n_inf


def sumsq_from_bins(b: List[int], n_nan: int, n_inf: int) -> float:
    """fl64 of the exact value sum_e b[e] * 2^(max(e,1) - 150) (item 3)."""
    if n_nan:
        return float("nan")
    if n_inf:
        return float("inf")
    total = Fraction(0)
    for e, v in enumerate(b):
        if v:
            total += Fraction(v) * Fraction(2) ** (max(e, 1) - 150)
    return float(total)  # Fraction -> float rounds to nearest even


def sumsq(xs: Iterable) -> float:
    """Exactly rounded sum of the float32 squares of every value in ``xs``."""
    parts = []
    for x in xs:
        parts.append(squares(x).ravel().astype(np.float64))
    if not parts:
        return 0.0
    s = np.concatenate(parts)
    if np.isnan(s).any():
        return float("nan")
    if np.isinf(s).any():
        return float("inf")
    return math.fsum(s.tolist())


def norm_from_sumsq(s: float) -> float:
    """fl32(sqrt(s)) for a float64 sum of squares (item 4)."""
    return float(np.float32(math.sqrt(s))) if s == s else float("nan")


def norm(xs: Iterable) -> Tuple[float, float]:
    """(sum of squares as float64, norm as float32) of every value in ``xs``."""
    s = sumsq(xs)
    return s, norm_from_sumsq(s)

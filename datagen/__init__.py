"""Seeded synthetic inputs for the token-logprob path.

This module produces *data only*: BF16 logit bit patterns, per-row sampling
parameters and target indices. It holds none of the log-probability
arithmetic, so both the CPU oracle and the GPU path can take their inputs from
it without sharing any computation.

Every row is generated from its own ``numpy.random.PCG64`` stream seeded by
``SeedSequence([seed, row])`` (or ``[seed, sequence, position]`` for the ragged
stress workload), so any single row can be regenerated cheaply and a full
batch can be filled by a thread pool in any order with identical bytes.

Shapes and distributions follow the workloads that the RL-Kernel pages
describe: Qwen3-8B logits over a real vocabulary of 151936 tokens padded to
152576 (page "Configurable H100 consistency runs", topology paragraph), BF16
model logits with float32 temperature scaling (same page, sampling paragraph),
and 8,192 active tokens per validation (page "H100 rollout context
parallelism", "Measured results"). The logits are synthetic normals; the pages
measured real model logits on a prompt set that is not available here.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Optional, Sequence

import numpy as np

# BF16 bit patterns used for padding and poison tests.
BF16_NEG_INF = 0xFF80
BF16_POS_INF = 0x7F80
BF16_NAN = 0x7FC0
BF16_MAX_FINITE = 0x7F7F

# Geometry of the Qwen3-8B vocabulary on the pages.
QWEN3_VOCAB_REAL = 151936
QWEN3_VOCAB_PADDED = 152576
N_SHARDS = 8

PAD_FILLS = {
    "neginf": BF16_NEG_INF,
    "nan": BF16_NAN,
    "posinf": BF16_POS_INF,
    "huge": BF16_MAX_FINITE,
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest BF16 (ties to even) and return the bits.

    NaN inputs map to the canonical quiet NaN 0x7FC0; overflow rounds to +-inf as
    IEEE round-to-nearest-even requires.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns to float32 (a 16-bit left shift)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(key: Sequence[int]) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(int(k) for k in key))))


def row_values(key: Sequence[int], vocab_real: int, sigma: float,
               spike: Optional[float] = None):
    """One row: (bf16 bits of the real columns, spike index or -1, uniform target).

    ``x = bf16_rne(sigma * N(0,1))`` in float32; when ``spike`` is given, ``spike``
    is added in float32 at one uniformly drawn index before rounding.
    """
    g = _rng(key)
    v = g.standard_normal(vocab_real, dtype=np.float32)
    v *= np.float32(sigma)
    spike_idx = -1
    if spike is not None:
        spike_idx = int(g.integers(0, vocab_real))
        v[spike_idx] += np.float32(spike)
    target = int(g.integers(0, vocab_real))
    return f32_to_bf16_bits(v), spike_idx, target


@dataclasses.dataclass
class Workload:
    """A batch of rows plus per-row sampling parameters (all host numpy arrays)."""

    name: str
    seed: int
    n_rows: int
    vocab_padded: int
    vocab_real: int
    row_stride: int
    sigma: float
    spike: Optional[float]
    temperature: np.ndarray  # float32 [n_rows]
    top_p: np.ndarray        # float32 [n_rows]
    top_k: np.ndarray        # int32 [n_rows]
    row_keys: list           # per-row seed keys
    pad_fill: int = BF16_NEG_INF
    seq_lengths: Optional[np.ndarray] = None  # ragged workloads only

    # ---- generation -------------------------------------------------------
    def row(self, i: int):
        return row_values(self.row_keys[i], self.vocab_real, self.sigma, self.spike)

    def fill_rows(self, out: np.ndarray, rows: Sequence[int], targets: Optional[np.ndarray] = None,
                  out_row_offset: int = 0):
        """Write rows ``rows`` into ``out[k]`` for k = index in ``rows`` (+offset)."""
        for k, i in enumerate(rows):
            bits, _, t = self.row(i)
            r = out[out_row_offset + k]
            r[: self.vocab_real] = bits
            r[self.vocab_real: self.vocab_padded] = self.pad_fill
            if self.row_stride > self.vocab_padded:
                r[self.vocab_padded: self.row_stride] = 0x7FC0  # never read
            if targets is not None:
                targets[out_row_offset + k] = t

    def generate(self, rows: Optional[Sequence[int]] = None, threads: Optional[int] = None,
                 out: Optional[np.ndarray] = None):
        """Return (logits uint16 [len(rows), row_stride], targets int64 [len(rows)])."""
        if rows is None:
            rows = range(self.n_rows)
        rows = list(rows)
        n = len(rows)
        if out is None:
            out = np.empty((n, self.row_stride), dtype=np.uint16)
        targets = np.empty(n, dtype=np.int64)
        if threads is None:
            threads = min(16, os.cpu_count() or 1)
        if n <= 64 or threads <= 1:
            self.fill_rows(out, rows, targets)
            return out, targets
        step = max(1, (n + 4 * threads - 1) // (4 * threads))
        chunks = [(s, rows[s:s + step]) for s in range(0, n, step)]
        with _cf.ThreadPoolExecutor(threads) as ex:
            futs = [ex.submit(self.fill_rows, out, ch, targets, s) for s, ch in chunks]
            for f in futs:
                f.result()
        return out, targets

    def checksum(self, rows: Sequence[int]) -> str:
        import hashlib
        h = hashlib.sha256()
        logits, targets = self.generate(rows, threads=1)
        h.update(logits.tobytes())
        h.update(targets.tobytes())
        return h.hexdigest()


def _const(n, v, dt):
    return np.full(n, v, dtype=dt)


def tiny(seed: int = 1001) -> Workload:
    """4 rows x vocab 1024 (real 1000), BF16 ~ N(0, 3^2), T = 1.0, pads = -inf."""
    n = 4
    return Workload("tiny", seed, n, 1024, 1000, 1024, 3.0, None,
                    _const(n, 1.0, np.float32), _const(n, 1.0, np.float32),
                    _const(n, -1, np.int32), [(seed, i) for i in range(n)])


def full(seed: int = 2002, n_rows: int = 8192) -> Workload:
    """Qwen3-8B-shaped full-vocab logp: 8192 x 152576 (real 151936), N(0, 2.5^2) + one +8 spike, T = 0.7."""
    return Workload("full", seed, n_rows, QWEN3_VOCAB_PADDED, QWEN3_VOCAB_REAL, QWEN3_VOCAB_PADDED,
                    2.5, 8.0, _const(n_rows, 0.7, np.float32), _const(n_rows, 1.0, np.float32),
                    _const(n_rows, -1, np.int32), [(seed, i) for i in range(n_rows)])


def nucleus(seed: int = 2002, n_rows: int = 8192) -> Workload:
    """The full-vocab logits with top-p 0.95 and top-k disabled (T = 0.7)."""
    w = full(seed, n_rows)
    w.name = "nucleus"
    w.top_p = _const(n_rows, 0.95, np.float32)
    return w


PER_REQUEST_T = (0.7, 1.0, 1.3)
PER_REQUEST_P = (0.95, 0.99)
PER_REQUEST_K = (-1, 128)


def per_request(seed: int = 4004, n_requests: int = 64, rows_per_request: int = 128) -> Workload:
    """64 requests x 128 rows; request r uses T, top-p, top-k chosen by r (all 12 combinations)."""
    n = n_requests * rows_per_request
    r = np.arange(n) // rows_per_request
    t = np.array(PER_REQUEST_T, dtype=np.float32)[r % 3]
    p = np.array(PER_REQUEST_P, dtype=np.float32)[(r // 3) % 2]
    k = np.array(PER_REQUEST_K, dtype=np.int32)[(r // 6) % 2]
    return Workload("per_request", seed, n, QWEN3_VOCAB_PADDED, QWEN3_VOCAB_REAL, QWEN3_VOCAB_PADDED,
                    2.5, None, t, p, k, [(seed, i) for i in range(n)])


def stress(seed: int = 5005, n_seqs: int = 64, max_len: int = 1024) -> Workload:
    """64 ragged sequences, lengths uniform in 1..1024, T = 0.7, top-p 0.95, top-k off."""
    lens = _rng((seed, 0xFFFF)).integers(1, max_len + 1, size=n_seqs)
    keys = [(seed, s, j) for s in range(n_seqs) for j in range(int(lens[s]))]
    n = len(keys)
    w = Workload("stress", seed, n, QWEN3_VOCAB_PADDED, QWEN3_VOCAB_REAL, QWEN3_VOCAB_PADDED,
                 2.5, None, _const(n, 0.7, np.float32), _const(n, 0.95, np.float32),
                 _const(n, -1, np.int32), keys)
    w.seq_lengths = lens.astype(np.int64)
    return w


def small(seed: int, n_rows: int, vocab_padded: int, vocab_real: int, sigma: float = 2.5,
          temperature=1.0, top_p=1.0, top_k=-1, spike: Optional[float] = None,
          row_stride: Optional[int] = None, pad: str = "neginf") -> Workload:
    """Free-form workload for parity and edge-case tests."""
    def arr(v, dt):
        a = np.asarray(v, dtype=dt)
        return np.broadcast_to(a, (n_rows,)).copy()
    return Workload(f"small{seed}", seed, n_rows, vocab_padded, vocab_real,
                    row_stride or vocab_padded, sigma, spike,
                    arr(temperature, np.float32), arr(top_p, np.float32), arr(top_k, np.int32),
                    [(seed, i) for i in range(n_rows)], pad_fill=PAD_FILLS[pad])


# --------------------------------------------------------------------------- gradient-norm inputs

NORM_MICROBENCH_N = 10_000_000  # page "H100 canonical CP backward validation", Timing and scope


def grad_values(seed: int, n: int, sigma: float = 1e-3, zero_frac: float = 0.0, chunk: int = 1 << 20) -> np.ndarray:
    """BF16-derived float32 gradient-like values: bf16_rne(sigma * N(0, 1)) widened
    to float32, with a fraction ``zero_frac`` of exact zeros. Chunk c of
    ``chunk`` values comes from ``SeedSequence([seed, c])`` so that any
    prefix is cheap to regenerate."""
    out = np.empty(n, dtype=np.float32)
    for c, lo in enumerate(range(0, n, chunk)):
        hi = min(n, lo + chunk)
        g = _rng((seed, c))
        v = (g.standard_normal(hi - lo, dtype=np.float32) * np.float32(sigma)).astype(np.float32)
        if zero_frac > 0:
            v[g.random(hi - lo) < zero_frac] = 0.0
        out[lo:hi] = bf16_bits_to_f32(f32_to_bf16_bits(v))
    return out


# --------------------------------------------------------------------------- LM-head inputs

QWEN3_D_MODEL = 4096  # Qwen3-8B hidden size


def linear_inputs(seed: int, n_rows: int, d_model: int, vocab_real: int, sigma_h: float = 1.0,
                  logit_sigma: float = 2.5, threads: Optional[int] = None):
    """BF16 hidden states ~ N(0, sigma_h^2) [n_rows, d_model] and a BF16 vocabulary
    projection ~ N(0, (logit_sigma / sqrt(d_model))^2) [vocab_real, d_model], so
    that the logits are roughly N(0, logit_sigma^2). Each block of 256 rows of
    each matrix comes from its own stream (seed, 0 or 1, block)."""
    hid = np.empty((n_rows, d_model), dtype=np.uint16)
    wt = np.empty((vocab_real, d_model), dtype=np.uint16)
    sw = logit_sigma / np.sqrt(d_model)
    step = 256

    def fill(kind, blk):
        dst, sig, n = (hid, sigma_h, n_rows) if kind == 0 else (wt, sw, vocab_real)
        lo, hi = blk * step, min(n, (blk + 1) * step)
        g = _rng((seed, kind, blk))
        v = g.standard_normal((hi - lo, d_model), dtype=np.float32) * np.float32(sig)
        dst[lo:hi] = f32_to_bf16_bits(v.astype(np.float32))

    jobs = [(0, b) for b in range((n_rows + step - 1) // step)] + \
           [(1, b) for b in range((vocab_real + step - 1) // step)]
    with _cf.ThreadPoolExecutor(max_workers=threads or min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda j: fill(*j), jobs))
    return hid, wt


def linear_exact_inputs(seed: int, n_rows: int, d_model: int, vocab_real: int, nnz: int = 80,
                        threads: Optional[int] = None):
    """Exactly summable BF16 inputs: hidden entries in {-3..3} / 4, and each
    vocabulary row with at most ``nnz`` entries of +-1/4 (``nnz`` uniform column
    draws; a repeated column keeps one entry; the rest 0). Every product is a
    multiple of 1/16, every partial sum of a row's dot product is such a
    multiple below 2^24/16 in magnitude (exact in float32 in any order), and
    every logit is a multiple of 1/16 of magnitude <= 3*nnz/16, which BF16
    holds exactly when 3*nnz <= 256. Each block of 256 rows comes from its own
    stream (seed, 10 or 11, block)."""
    hid = np.empty((n_rows, d_model), dtype=np.uint16)
    wt = np.zeros((vocab_real, d_model), dtype=np.uint16)
    hv = f32_to_bf16_bits(np.arange(-3, 4, dtype=np.float32) / 4)       # index v+3 -> bits of v/4
    qv = f32_to_bf16_bits(np.array([-0.25, 0.25], dtype=np.float32))
    step = 256

    def fill(kind, blk):
        n = n_rows if kind == 0 else vocab_real
        lo, hi = blk * step, min(n, (blk + 1) * step)
        g = _rng((seed, 10 + kind, blk))
        if kind == 0:
            hid[lo:hi] = hv[g.integers(0, 7, (hi - lo, d_model))]
        else:
            cols = g.integers(0, d_model, (hi - lo, nnz))
            vals = qv[g.integers(0, 2, (hi - lo, nnz))]
            wt[np.arange(lo, hi)[:, None], cols] = vals

    jobs = [(0, b) for b in range((n_rows + step - 1) // step)] + \
           [(1, b) for b in range((vocab_real + step - 1) // step)]
    with _cf.ThreadPoolExecutor(max_workers=threads or min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda j: fill(*j), jobs))
    return hid, wt

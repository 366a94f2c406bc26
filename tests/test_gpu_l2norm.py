"""GPU parity of the order-independent FP32 L2 norm (include/rlk_norm.h)
against the CPU oracle (oracle/l2norm.py).

Passage: RL-Kernel page "H100 canonical CP backward validation", Change
section (FP32 gradient squares summed in integer exponent bins before the
distributed reduction) and Timing and scope section (10M-element BF16-derived
FP32 microbenchmark).

The result is uniquely defined (the exact sum of the float32 squares rounded
once to float64, and fl32 of its square root), so the bar is bit equality of
the sum and the norm, exact equality of the value the accumulator words
encode (the words themselves may spread that value differently), and exact
NaN/inf counts.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import datagen
import invariant_token_log_fp32_amd as rlk
from oracle import l2norm as L

from gpu_util import say, to_host

pytestmark = pytest.mark.gpu


def dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


def exact_value(words):
    """Exact sum encoded by accumulator words (finite part)."""
    return sum((Fraction(int(v)) * Fraction(2) ** (max(e, 1) - 150) for e, v in enumerate(words[:256]) if v),
               Fraction(0))


def gpu_norm(xs):
    """Values from the one-launch rlk_l2norm (single tensor) and the words from
    zero + accumulate + finalize; both must give the same values."""
    import torch
    dev = "cuda:0"
    bins = torch.empty(rlk.NORM_BIN_WORDS, dtype=torch.int64, device=dev)
    s2, n2 = rlk.l2norm(list(xs) if isinstance(xs, (list, tuple)) else [xs], workspace=bins)
    torch.cuda.synchronize()
    words = to_host(bins).view(np.uint64).copy()
    s2, n2 = float(to_host(s2)[0]), float(to_host(n2)[0])
    if isinstance(xs, (list, tuple)):
        return s2, n2, words
    ws = torch.zeros(rlk.NORM_BIN_WORDS, dtype=torch.int64, device=dev)
    s1, n1 = rlk.l2norm(xs, workspace=ws)
    torch.cuda.synchronize()
    assert not to_host(ws).any(), "rlk_l2norm must leave its workspace all-zero"
    s1, n1 = float(to_host(s1)[0]), float(to_host(n1)[0])
    assert (s1 == s2 or (math.isnan(s1) and math.isnan(s2))) and (n1 == n2 or (math.isnan(n1) and math.isnan(n2)))
    return s1, n1, words


def check(xs_host, what, xs_dev=None):
    xs_dev = xs_dev if xs_dev is not None else [dev_f32(a) for a in xs_host]
    s, n, b = gpu_norm(xs_dev if len(xs_dev) > 1 else xs_dev[0])
    want_s, want_n = L.norm(xs_host)
    wb, wnan, winf = L.bins(xs_host)
    assert int(b[256]) == wnan and int(b[257]) == winf and np.all(b[258:] == 0), f"{what}: counts"
    assert exact_value(b) == exact_value(wb), f"{what}: the accumulator's exact value differs"
    if math.isnan(want_s):
        assert math.isnan(s) and math.isnan(n), what
    else:
        assert s == want_s and n == want_n, f"{what}: got ({s!r}, {n!r}) want ({want_s!r}, {want_n!r})"
    return s, n, b


def wide_values(n, rng, lo=-80, hi=64):
    mant = rng.uniform(1.0, 2.0, n)
    exp = rng.integers(lo, hi, n)
    v = (mant * np.exp2(exp) * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    v[rng.random(n) < 0.05] = 0.0
    return v


def test_microbenchmark_size():
    """10M BF16-derived FP32 values (the pages' microbenchmark size)."""
    say("case: 10M BF16-derived values")
    x = datagen.grad_values(7, datagen.NORM_MICROBENCH_N)
    check([x], "10M")


def test_ragged_sizes_and_offsets():
    import torch
    rng = np.random.default_rng(3)
    buf_h = wide_values(1_300_000, rng)
    buf = dev_f32(buf_h)
    for n in (1, 2, 3, 4, 5, 7, 17, 1000, 4097, 1_234_567):
        for off in (0, 1, 2, 3):
            say(f"case: n {n} offset {off}")
            check([buf_h[off:off + n]], f"n {n} offset {off}", [buf[off:off + n]])


def test_rounding_of_the_final_sum():
    """Many small arrays with wide exponent spreads: the exact sums carry far
    more than 53 bits, which exercises the float64 rounding and the square root."""
    rng = np.random.default_rng(17)
    for trial in range(150):
        n = int(rng.integers(1, 3000))
        lo = int(rng.integers(-75, 0))
        x = wide_values(n, rng, lo, lo + int(rng.integers(1, 70)))
        check([x], f"trial {trial}")


def test_tensor_lists_and_partitions():
    rng = np.random.default_rng(23)
    parts = [wide_values(int(rng.integers(0, 50_000)), rng) for _ in range(9)]
    whole = np.concatenate(parts)
    s0, n0, b0 = check([whole], "whole")
    s1, n1, b1 = check(parts, "parts")
    s2, n2, b2 = check(parts[::-1], "parts reversed")
    assert (s0, n0) == (s1, n1) == (s2, n2) and exact_value(b0) == exact_value(b1) == exact_value(b2)


def test_special_values():
    base = datagen.grad_values(5, 100_000)
    for what, pos, val in (("nan", 77, np.nan), ("inf", 99_999, np.inf), ("-inf", 0, -np.inf),
                           ("overflowing square", 5000, 2.0 ** 64), ("zero", 3, 0.0),
                           ("subnormal square", 11, 2.0 ** -70), ("square rounding to zero", 12, 2.0 ** -75)):
        x = base.copy()
        x[pos] = val
        say(f"case: {what}")
        check([x], what)
    check([np.zeros(1000, np.float32)], "all zeros")


def test_large_array_bins_add_up():
    """2^28 values (1 GiB): the exact value of the whole's accumulator equals
    the sum of its quarters' values, the finalised values equal the oracle's
    value of those words, and repeat calls give identical words."""
    import torch
    n = 1 << 28
    say("case: 2^28 values")
    x = torch.randn(n, generator=torch.Generator(device="cuda:0").manual_seed(3), device="cuda:0")
    x = x.to(torch.bfloat16).to(torch.float32) * 1e-3
    s, nn, b = gpu_norm(x)
    s2, nn2, b2 = gpu_norm(x)
    assert (s, nn) == (s2, nn2) and np.array_equal(b, b2)
    total = Fraction(0)
    for q in range(4):
        _, _, bq = gpu_norm(x[q * (n // 4):(q + 1) * (n // 4)])
        total += exact_value(bq)
    assert total == exact_value(b)
    want = float(total)
    assert s == want and nn == L.norm_from_sumsq(want)

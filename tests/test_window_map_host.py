"""Host check of the support window's slot arithmetic (no GPU).

The nucleus kernel counts each BF16 token into a window of classes with
magnitudes in [2^-24, 4096) of both signs, interleaved (slot
2 * (m - 0x3380) + sign), plus a class for +-0. Two tokens packed in a 32-bit
word get their slots from three packed 16-bit integer instructions (shift
right by 15, multiply-add 2 * b + sign, subtract 2 * 0x3380); a slot below
9216 means "in the window". This emulates those instructions' 16-bit
wrap-around arithmetic on all 65536 patterns and checks:
- the packed result equals the scalar definition for every in-window pattern
  and is 9216 or more for every pattern outside (zeros, tiny and huge
  magnitudes, infinities, NaN), in both halves of a word;
- visiting the slots in the kernel's rank order (positive slots from the top,
  the zero class, negative slots from the top) lists the in-window values in
  strictly decreasing order, each exactly once.
The classes are the BF16 values themselves (page "Configurable H100
consistency runs", sampling paragraph: support over the real vocabulary; ties
by value are one class).
"""
import numpy as np

import datagen

MAG_LO = 0x3380
N_MAG = 4608
WIN = 2 * N_MAG


def packed_slots(words):
    """v_pk_lshrrev_b16 15 / v_pk_mad_u16 (w, 2, sign) / v_pk_sub_u16 0x6700,
    each on the two 16-bit halves independently, modulo 2^16."""
    lo = (words & 0xFFFF).astype(np.uint32)
    hi = (words >> 16).astype(np.uint32)

    def half(b):
        sgn = b >> 15
        u = (b * 2 + sgn) & 0xFFFF
        return (u - 2 * MAG_LO) & 0xFFFF

    return half(lo), half(hi)


def scalar_slot(b):
    m = b & 0x7FFF
    if m == 0:
        return "zero"
    k = m - MAG_LO
    return 2 * k + (b >> 15) if 0 <= k < N_MAG else None


def test_packed_slots_equal_the_scalar_map_on_every_pattern():
    pats = np.arange(65536, dtype=np.uint32)
    # every pattern in the low half with a varying high half, and the reverse
    words = pats | (((pats * 40503) & 0xFFFF) << 16)
    for words_, which in ((words, 0), (((pats << 16) | ((pats * 40503) & 0xFFFF)), 1)):
        lo, hi = packed_slots(words_)
        got = lo if which == 0 else hi
        for b in range(65536):
            want = scalar_slot(b)
            g = int(got[b])
            if want is None or want == "zero":
                assert g >= WIN, hex(b)
            else:
                assert g == want, hex(b)


def test_rank_order_is_value_order():
    ranks = []
    for k in range(N_MAG - 1, -1, -1):           # positive slots, largest magnitude first
        ranks.append(MAG_LO + k)
    ranks.append(0)                                # the zero class
    for k in range(N_MAG):                         # negative slots, smallest magnitude first
        ranks.append(0x8000 | (MAG_LO + k))
    vals = datagen.bf16_bits_to_f32(np.array(ranks, dtype=np.uint16)).astype(np.float64)
    assert np.all(np.diff(vals) < 0)
    assert len(ranks) == WIN + 1
    inside = [b for b in range(65536) if scalar_slot(b) not in (None, "zero")]
    assert sorted(inside) == sorted(b for b in ranks if b != 0)
    assert vals[0] == 4080.0 and vals[-1] == -4080.0
    assert vals[N_MAG - 1] == 2.0 ** -24 and vals[N_MAG + 1] == -(2.0 ** -24)


def test_signed_16_bit_maximum_of_patterns_is_the_row_maximum():
    """The count's row maximum: a signed 16-bit maximum over the raw BF16
    patterns of a row whose tokens lie in the window, are +-0 or -inf. When it
    is >= 0 (the row holds +0 or a positive token) it must be the pattern of
    the row's largest value; when it is negative the kernel scans the window
    instead. Checked on every window pattern as a row of one token beside a
    random row, and on random rows that mix signs, zeros and -inf."""
    rng = np.random.default_rng(5)
    window = np.array([b for b in range(65536) if scalar_slot(b) not in (None,)], dtype=np.uint16)
    pool = np.concatenate([window, np.array([0x0000, 0x8000, 0xFF80], np.uint16)])

    def check(row):
        m = int(row.view(np.int16).max())
        vals = datagen.bf16_bits_to_f32(row).astype(np.float64)
        if m >= 0:
            want = float(vals.max())
            got = float(datagen.bf16_bits_to_f32(np.array([m], np.uint16))[0])
            assert got == want, (hex(m), got, want)
        else:
            assert vals.max() <= 0.0
    base = rng.choice(pool, 64)
    for b in pool:
        row = base.copy()
        row[int(rng.integers(0, 64))] = b
        check(row)
    for _ in range(2000):
        n = int(rng.integers(1, 200))
        row = rng.choice(pool, n)
        if rng.random() < 0.3:
            row = row[(row & 0x8000) != 0] if np.any((row & 0x8000) != 0) else row
        check(row)

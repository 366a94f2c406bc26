"""Host emulation of the L2 norm finalize's exact integer sum (64-bit lanes,
shuffle trees, 64-bit limbs with carry counts), checked against the plain
big-integer sum of the bins: bin e weighs 2^(max(e,1) - 1) units of 2^-149.

Every value is masked to 64 bits as on the GPU, so a lost carry or a wrong
shift or limb index shows up as a different total. Defining passage: RL-Kernel
page "H100 canonical CP backward validation", Change section (integer exponent
bins, exact in any reduction order)."""
import random

M64 = (1 << 64) - 1


def bin_offset(e):
    return e - 1 if e > 0 else 0


def add_shl128(a_lo, a_hi, v_lo, v_hi, sh):
    s_lo = (v_lo << sh) & M64
    s_hi = (((v_hi << sh) & M64) | (v_lo >> (64 - sh))) if sh else v_hi
    t = (a_lo + s_lo) & M64
    a_hi = (a_hi + s_hi + (1 if t < s_lo else 0)) & M64
    return t, a_hi


def emulate(bins):
    lo = [0] * 64
    hi = [0] * 64
    for j in range(64):
        o = bin_offset(4 * j)
        for i in range(4):
            lo[j], hi[j] = add_shl128(lo[j], hi[j], bins[4 * j + i], 0, bin_offset(4 * j + i) - o)
    d = 1
    while d < 8:
        src_lo, src_hi = lo[:], hi[:]
        for j in range(64):
            if j & (2 * d - 1) == 0:
                lo[j], hi[j] = add_shl128(lo[j], hi[j], src_lo[j + d], src_hi[j + d],
                                          bin_offset(4 * (j + d)) - bin_offset(4 * j))
        d <<= 1
    s_lo = [[0] * 6 for _ in range(64)]
    s_c = [[0] * 6 for _ in range(64)]
    for j in range(0, 64, 8):
        o = bin_offset(4 * j)
        limb0, sh = o >> 6, o & 63
        q0 = (lo[j] << sh) & M64
        q1 = ((((hi[j] << sh) & M64) | (lo[j] >> (64 - sh))) if sh else hi[j])
        q2 = (hi[j] >> (64 - sh)) if sh else 0
        for k, q in ((limb0, q0), (limb0 + 1, q1), (limb0 + 2, q2)):
            s_lo[j][k] = q
    d = 8
    while d < 64:
        src_lo = [r[:] for r in s_lo]
        src_c = [r[:] for r in s_c]
        for j in range(64):
            if j & (2 * d - 1) == 0:
                for k in range(6):
                    t = (s_lo[j][k] + src_lo[j + d][k]) & M64
                    s_c[j][k] = (s_c[j][k] + src_c[j + d][k] + (1 if t < src_lo[j + d][k] else 0)) & M64
                    s_lo[j][k] = t
        d <<= 1
    total, carry = 0, 0
    for k in range(6):
        t = (s_lo[0][k] + carry) & M64
        total |= t << (64 * k)
        carry = (s_c[0][k] + (1 if t < carry else 0)) & M64
    assert carry == 0
    return total


def plain(bins):
    return sum(b << bin_offset(e) for e, b in enumerate(bins))


def test_random_and_extreme_bins():
    rng = random.Random(5)
    cases = [[0] * 256, [(1 << 63) - 1] * 256, [1] * 256]
    for _ in range(60):
        kind = rng.randrange(4)
        if kind == 0:
            bins = [rng.getrandbits(63) for _ in range(256)]
        elif kind == 1:
            bins = [rng.getrandbits(rng.randrange(1, 64)) if rng.random() < 0.1 else 0 for _ in range(256)]
        elif kind == 2:
            bins = [(1 << 63) - 1 - rng.getrandbits(8) for _ in range(256)]
        else:
            bins = [0] * 256
            for e in rng.sample(range(256), 3):
                bins[e] = rng.getrandbits(63)
        cases.append(bins)
    for bins in cases:
        assert emulate(bins) == plain(bins)


def test_each_bin_alone():
    for e in range(256):
        bins = [0] * 256
        bins[e] = (1 << 63) - 1
        assert emulate(bins) == plain(bins), e

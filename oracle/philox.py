"""Philox counter-based generator, written for the oracle (test infrastructure).

The VASE summary (gist.science 2606.03928, §2.B) replaces deterministic top-k
with weighted random sampling but names no generator.  The random draws are
fixed here by a counter-based generator so that two independent
implementations (this one and the device one) can agree word for word:
Philox-4xW with R rounds, from Salmon, Moraes, Dror and Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3" (SC'11).  One round maps the counter
(c0, c1, c2, c3) under key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

and the key is bumped by the Weyl constants (W0, W1) before every round after
the first.  The code is generic in the word width W so that the 64-bit
instance can be checked against numpy's own Philox4x64-10 bit generator; the
32-bit instance is the one the sampling uses.

Only tests, the smoke check and the CPU baseline leg of the benchmark may
import this module.
"""
import numpy as np

# Multipliers and Weyl increments of the SC'11 paper, per word width.
MULTIPLIERS = {
    32: (0xD2511F53, 0xCD9E8D57),
    64: (0xD2E7470EE14C6C93, 0xCA5A826395121157),
}
WEYL = {
    32: (0x9E3779B9, 0xBB67AE85),
    64: (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B),
}

_U64 = np.uint64


def _mask(width):
    return _U64((1 << width) - 1)


def mulhilo(a, b, width):
    """Full product of two W-bit words, returned as (high word, low word).

    a and b are uint64 arrays (or scalars) holding W-bit values."""
    a = np.asarray(a, dtype=_U64)
    b = np.asarray(b, dtype=_U64)
    if width == 32:
        p = a * b  # < 2**64, exact in uint64
        return p >> _U64(32), p & _U64(0xFFFFFFFF)
    if width == 64:
        # 128-bit product from four 32x32 partial products.
        m32 = _U64(0xFFFFFFFF)
        a0, a1 = a & m32, a >> _U64(32)
        b0, b1 = b & m32, b >> _U64(32)
        p00 = a0 * b0
        p01 = a0 * b1
        p10 = a1 * b0
        p11 = a1 * b1
        mid = (p00 >> _U64(32)) + (p01 & m32) + (p10 & m32)  # < 3 * 2**32
        lo = (p00 & m32) | ((mid & m32) << _U64(32))
        hi = p11 + (p01 >> _U64(32)) + (p10 >> _U64(32)) + (mid >> _U64(32))
        return hi, lo
    raise ValueError("width must be 32 or 64")


def philox4(counter, key, width=32, rounds=10):
    """Philox-4xW-R block function.

    counter: four arrays (or scalars) of W-bit words; key: two W-bit words
    (arrays or scalars, broadcast against the counter).  Returns the four
    output words as uint64 arrays."""
    m0, m1 = (_U64(v) for v in MULTIPLIERS[width])
    w0, w1 = (_U64(v) for v in WEYL[width])
    msk = _mask(width)
    c0, c1, c2, c3 = (np.asarray(c, dtype=_U64) & msk for c in counter)
    k0, k1 = (np.asarray(k, dtype=_U64) & msk for k in key)
    with np.errstate(over="ignore"):
        for r in range(rounds):
            if r:
                k0 = (k0 + w0) & msk
                k1 = (k1 + w1) & msk
            hi0, lo0 = mulhilo(m0, c0, width)
            hi1, lo1 = mulhilo(m1, c2, width)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 on uint32-valued inputs; returns four uint64 arrays."""
    return philox4((c0, c1, c2, c3), (k0, k1), width=32, rounds=10)


def seed_key(seed):
    """Split a 64-bit seed into the two 32-bit key words (low, high)."""
    seed = int(seed) & ((1 << 64) - 1)
    return seed & 0xFFFFFFFF, seed >> 32

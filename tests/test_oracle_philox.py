"""Pins for the oracle's Philox generator and exponential variates."""
import math

import numpy as np
import pytest
from scipy import stats

from oracle import philox4, philox4x32_10, mulhilo, exp_variate, philox_word0, seed_key


def test_philox4x64_matches_numpy_bit_generator():
    # numpy.random.Philox is Philox4x64-10; it bumps the counter by one
    # before each block, so block n of counter c is philox(c + n + 1).
    rng = np.random.default_rng(7)
    for _ in range(20):
        key = [int(v) for v in rng.integers(0, 2**63, size=2, dtype=np.uint64)]
        ctr = [int(v) for v in rng.integers(0, 2**62, size=4, dtype=np.uint64)]
        bg = np.random.Philox(key=key, counter=ctr)
        raw = bg.random_raw(12)
        for blk in range(3):
            c = list(ctr)
            c[0] += blk + 1
            out = philox4(tuple([v] for v in c), tuple(key), width=64, rounds=10)
            got = [int(o[0]) for o in out]
            assert got == [int(x) for x in raw[4 * blk:4 * blk + 4]]


def test_mulhilo32_against_python_integers():
    rng = np.random.default_rng(1)
    a = rng.integers(0, 2**32, size=1000, dtype=np.uint64)
    b = rng.integers(0, 2**32, size=1000, dtype=np.uint64)
    hi, lo = mulhilo(a, b, 32)
    for x, y, h, l in zip(a, b, hi, lo):
        p = int(x) * int(y)
        assert int(h) == p >> 32 and int(l) == p & 0xFFFFFFFF
    hi, lo = mulhilo(a << np.uint64(31), b << np.uint64(30), 64)
    for x, y, h, l in zip(a << np.uint64(31), b << np.uint64(30), hi, lo):
        p = int(x) * int(y)
        assert int(h) == p >> 64 and int(l) == p & (2**64 - 1)


def test_philox4x32_words_uniform():
    # word 0 over the (row, head, layer, batch) counter grid used by selection
    t = np.arange(1 << 18, dtype=np.uint64)
    words = []
    for head in range(2):
        for layer in range(2):
            w = philox4x32_10(t, head, layer, 0, *seed_key(12345))
            words.append(np.stack(w))
    allw = np.concatenate(words, axis=1)          # [4][2**20]
    for row in allw:
        counts = np.bincount((row >> np.uint64(24)).astype(np.int64), minlength=256)
        chi2 = ((counts - counts.mean()) ** 2 / counts.mean()).sum()
        assert stats.chi2.sf(chi2, 255) > 1e-3
        bits = np.unpackbits(row.astype(">u4").view(np.uint8)).reshape(-1, 32).mean(axis=0)
        assert np.all(np.abs(bits - 0.5) < 0.005)


def test_philox4x32_avalanche_and_key_sensitivity():
    rng = np.random.default_rng(3)
    base = rng.integers(0, 2**32, size=(4, 4096), dtype=np.uint64)
    out0 = philox4x32_10(*base, 11, 22)[0]
    for word in range(4):
        for bit in (0, 13, 31):
            flipped = base.copy()
            flipped[word] ^= np.uint64(1 << bit)
            out1 = philox4x32_10(*flipped, 11, 22)[0]
            diff = np.unpackbits((out0 ^ out1).astype(">u4").view(np.uint8)).mean()
            assert abs(diff - 0.5) < 0.02
    out_k = philox4x32_10(*base, 12, 22)[0]
    assert np.mean(out_k == out0) < 1e-3


def test_seed_key_split():
    assert seed_key(0) == (0, 0)
    assert seed_key(0x123456789ABCDEF0) == (0x9ABCDEF0, 0x12345678)


def test_exp_variate_end_points_and_law():
    assert exp_variate(np.array([2**32 - 1.0]))[0] == 0.0
    assert exp_variate(np.array([0.0]))[0] == pytest.approx(32 * math.log(2), rel=1e-15)
    x = philox_word0(np.arange(200000), 0, 0, 0, 99)
    e = exp_variate(x)
    assert e.min() >= 0.0
    assert abs(e.mean() - 1.0) < 0.01
    assert stats.kstest(e, "expon").pvalue > 1e-3
    # full relative accuracy for words near 2**32 - 1 (tiny E): with
    # y = m / 2**32, -ln(1 - y) = y + y**2/2 + y**3/3 + O(y**4)
    m = np.array([1.0, 10.0, 1000.0, 65536.0])
    y = m / 2**32
    e_small = exp_variate(2**32 - 1 - m)
    assert np.allclose(e_small, y + y * y / 2 + y**3 / 3, rtol=1e-13, atol=0)


def test_weyl_increments_closed_forms():
    # The key increments are the leading fraction bits of the golden ratio
    # and of sqrt(3) (SC'11, the Philox key schedule); the 32-bit ones are
    # the high words of the 64-bit ones, which the numpy check above fixes.
    from decimal import Decimal, getcontext
    from oracle.philox import WEYL
    getcontext().prec = 60
    phi_frac = (Decimal(5).sqrt() - 1) / 2
    sqrt3_frac = Decimal(3).sqrt() - 1
    for width in (32, 64):
        scale = Decimal(2) ** width
        assert WEYL[width][0] == int(phi_frac * scale)
        assert WEYL[width][1] == int(sqrt3_frac * scale)
    assert WEYL[32] == tuple(w >> 32 for w in WEYL[64])


def test_philox4x32_10_known_answer_vectors():
    # The published known-answer vectors of Philox4x32-10 (Random123, the
    # library of Salmon et al., SC'11): all-zero, all-ones and the pi-digit
    # counter/key.  They pin both 32-bit multipliers, the Weyl increments,
    # the word order of a round and the round count at once.
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")
    vecs = json.load(open(path))["vectors"]
    assert len(vecs) == 3
    for v in vecs:
        c = [int(x, 16) for x in v["counter"]]
        k = [int(x, 16) for x in v["key"]]
        got = [int(w) for w in philox4x32_10(*c, *k)]
        assert got == [int(x, 16) for x in v["out"]], v
    # a plausible slip anywhere in the round changes every vector
    from oracle import philox as ph
    c = [int(x, 16) for x in vecs[2]["counter"]]
    k = [int(x, 16) for x in vecs[2]["key"]]
    want = [int(x, 16) for x in vecs[2]["out"]]
    assert [int(w) for w in ph.philox4(c, k, width=32, rounds=9)] != want
    swapped = ph.philox4([c[2], c[1], c[0], c[3]], k, width=32, rounds=10)
    assert [int(w) for w in swapped] != want

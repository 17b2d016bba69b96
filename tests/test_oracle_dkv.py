"""Pins of the VASE-DKV oracle (oracle/dkv.py) against mathematics that does
not go through its own code path: QR and SVD leverage (library routines of a
different algorithm), closed forms, invariances, the normal law."""
import math

import numpy as np
import pytest
from scipy import stats

from oracle import dkv
from oracle.philox import philox4x32_10, seed_key


def rng(s):
    return np.random.default_rng(s)


# ---------------------------------------------------------------- generator
def test_box_muller_word_roles():
    # x0 = 2^32 - 1 gives u1 = 1, radius 0: both outputs are exactly zero.
    z0, z1 = dkv.box_muller(np.array([2**32 - 1]), np.array([12345]))
    assert z0[0] == 0.0 and z1[0] == 0.0
    # x1 = 0 gives angle 0: z0 = radius, z1 = 0.
    z0, z1 = dkv.box_muller(np.array([2**31 - 1]), np.array([0]))
    assert z1[0] == 0.0 and z0[0] == pytest.approx(math.sqrt(-2 * math.log(0.5)), rel=1e-15)
    # x1 = 2^30 gives a quarter turn: z0 = 0 (to rounding), z1 = radius.
    z0, z1 = dkv.box_muller(np.array([2**31 - 1]), np.array([2**30]))
    assert abs(z0[0]) < 1e-15 and z1[0] == pytest.approx(math.sqrt(2 * math.log(2)), rel=1e-15)


def test_gaussian_uses_philox_words_of_its_counter():
    n = 10
    bits = dkv.gaussian_bf16(n, seed=77, c1=5, c2=9)
    k0, k1 = seed_key(77)
    for i in range(n):
        p = i // 2
        x = philox4x32_10(np.uint64(p), np.uint64(5), np.uint64(9), np.uint64(0),
                          np.uint64(k0), np.uint64(k1))
        u1 = (float(x[0]) + 1) / 2**32
        u2 = float(x[1]) / 2**32
        rad = math.sqrt(-2 * math.log(u1))
        z = rad * (math.cos if i % 2 == 0 else math.sin)(2 * math.pi * u2)
        want = dkv.bf16_round_bits(np.float32(z))
        assert bits[i] == want


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -2.5], np.float32)
    got = dkv.bf16_bits_to_f64(dkv.bf16_round_bits(f))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1) wins;
    # 1 + 3*2^-8 ties between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6.
    assert list(got) == [1.0, 1.0, 1.0 + 2**-6, 1.0 + 2**-7, -2.5]


def test_gaussian_law():
    z = dkv.bf16_bits_to_f64(dkv.gaussian_bf16(200000, seed=3, c1=1, c2=2))
    assert abs(z.mean()) < 5 / math.sqrt(len(z))
    assert abs(z.var() - 1) < 5 * math.sqrt(2 / len(z)) + 2e-3   # bf16 rounding adds ~1e-5
    # bf16 keeps 8 bits: compare with the normal law at a coarse resolution
    ks = stats.kstest(z + rng(0).uniform(-1, 1, len(z)) * np.abs(z) * 2**-9, "norm")
    assert ks.pvalue > 1e-3


def test_gaussian_streams_differ_by_counter():
    a = dkv.gaussian_bf16(1000, seed=3, c1=1, c2=2)
    b = dkv.gaussian_bf16(1000, seed=3, c1=2, c2=2)
    c = dkv.gaussian_bf16(1000, seed=4, c1=1, c2=2)
    assert (a != b).mean() > 0.9 and (a != c).mean() > 0.9


# ----------------------------------------------------------------- leverage
def qr_leverage(Y):
    Q, _ = np.linalg.qr(Y)
    return (Q * Q).sum(1)


def svd_leverage(A, tol=1e-10):
    U, s, _ = np.linalg.svd(A, full_matrices=False)
    k = int((s > tol * s[0]).sum())
    return (U[:, :k] ** 2).sum(1), k


@pytest.mark.parametrize("T,d,r", [(40, 8, 4), (300, 16, 16), (1000, 64, 32)])
def test_leverage_matches_qr(T, d, r):
    g = rng(T)
    K, V = g.normal(size=(T, d)), g.normal(size=(T, d))
    G = g.normal(size=(2 * d, r))
    l = dkv.dkv_score(K, V, G)
    np.testing.assert_allclose(l, qr_leverage(np.concatenate([K, V], 1) @ G), atol=1e-12)
    assert abs(l.sum() - r) < 1e-9
    assert l.min() >= -1e-15 and l.max() <= 1 + 1e-12


def test_full_sketch_gives_leverage_of_kv_rows():
    # r >= rank([K|V]): the sketch keeps the whole column space, so the
    # scores are the exact leverage of the concatenated rows (SVD).
    g = rng(1)
    T, d = 120, 6
    K, V = g.normal(size=(T, d)), g.normal(size=(T, d)) * 3
    G = g.normal(size=(2 * d, 2 * d + 4))
    lev, k = svd_leverage(np.concatenate([K, V], 1))
    assert k == 2 * d
    np.testing.assert_allclose(dkv.dkv_score(K, V, G), lev, atol=1e-9)


def test_only_the_sketch_subspace_matters():
    g = rng(2)
    K, V = g.normal(size=(200, 8)), g.normal(size=(200, 8))
    G = g.normal(size=(16, 5))
    B = g.normal(size=(5, 5)) + 3 * np.eye(5)
    np.testing.assert_allclose(dkv.dkv_score(K, V, G), dkv.dkv_score(K, V, G @ B), atol=1e-10)


def test_value_half_counts():
    # the V half of the row enters the score: zeroing the key half leaves the
    # leverage of the value rows
    g = rng(3)
    T, d = 150, 5
    V = g.normal(size=(T, d))
    G = g.normal(size=(2 * d, 2 * d))
    lev, _ = svd_leverage(V)
    np.testing.assert_allclose(dkv.dkv_score(np.zeros((T, d)), V, G), lev, atol=1e-9)
    lev_k, _ = svd_leverage(V[:, ::-1] * 2)
    np.testing.assert_allclose(dkv.dkv_score(V[:, ::-1] * 2, np.zeros((T, d)), G), lev_k, atol=1e-9)


def test_two_rows_one_column_closed_form():
    a1, a2 = np.array([[1.0, 2.0]]), np.array([[3.0, -1.0]])
    K = np.concatenate([a1[:, :1], a2[:, :1]])
    V = np.concatenate([a1[:, 1:], a2[:, 1:]])
    G = np.array([[0.5], [2.0]])
    y1, y2 = 1.0 * 0.5 + 2.0 * 2.0, 3.0 * 0.5 - 1.0 * 2.0
    want = np.array([y1 * y1, y2 * y2]) / (y1 * y1 + y2 * y2)
    np.testing.assert_allclose(dkv.dkv_score(K, V, G), want, rtol=1e-14)


def test_isolated_direction_has_leverage_one():
    # one token whose row is orthogonal to every other row
    g = rng(4)
    T, d = 64, 8
    K = np.zeros((T, d)); V = np.zeros((T, d))
    K[:, :4] = g.normal(size=(T, 4))
    K[17] = 0.0
    V[17, 0] = 5.0
    G = g.normal(size=(2 * d, 12))
    l = dkv.dkv_score(K, V, G)
    assert abs(l[17] - 1.0) < 1e-10
    assert abs(l.sum() - 5.0) < 1e-9          # rank 4 + 1


def test_rank_deficient_rows_drop_directions():
    # rank-3 rows, 10 sketch columns: 7 directions are dropped and the scores
    # are the leverage of the rank-3 row space
    g = rng(5)
    T, d = 90, 6
    A = g.normal(size=(T, 3)) @ g.normal(size=(3, 2 * d))
    G = g.normal(size=(2 * d, 10))
    l = dkv.dkv_score(A[:, :d], A[:, d:], G)
    lev, k = svd_leverage(A)
    assert k == 3
    assert abs(l.sum() - 3) < 1e-6
    np.testing.assert_allclose(l, lev, atol=1e-6)


def test_zero_cache_scores_zero():
    assert not dkv.dkv_score(np.zeros((10, 4)), np.zeros((10, 4)), np.ones((8, 3))).any()


def test_duplicate_rows_share_leverage():
    g = rng(6)
    K, V = g.normal(size=(50, 4)), g.normal(size=(50, 4))
    K[10], V[10] = K[3], V[3]
    G = g.normal(size=(8, 8))
    l = dkv.dkv_score(K, V, G)
    assert abs(l[3] - l[10]) < 1e-12
    # removing the copy moves the shared direction's weight back to one row
    keep = [i for i in range(50) if i != 10]
    l2 = dkv.dkv_score(K[keep], V[keep], G)
    assert l2[3] > l[3]

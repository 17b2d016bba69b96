"""Pins of the cross-layer factorisation / selective reconstruction oracle
(oracle/xkv.py): the page's storage formula, exact reconstruction at full
rank and for exactly shared structure, a closed-form rank-1 case, optimality
against other subspaces, landmark and chunk-score definitions by brute
force, the selection rule, and the exact merge of two attention parts."""
import math

import numpy as np
import pytest

import oracle
from oracle import xkv


def rng(s):
    return np.random.default_rng(s)


def test_memory_formula_and_page_ratio():
    # xKV summary §2.2: W caches of T x d numbers become T x r + W x r x d
    assert xkv.memory_floats(100, 4, 8, 16) == (100 * 8 + 4 * 8 * 16, 4 * 100 * 16)
    stored, full = xkv.memory_floats(32768, 4, 64, 128)
    assert full / stored == pytest.approx(7.877, abs=1e-3)       # the page's "up to 8x"
    A, Bs = xkv.clf([rng(0).normal(size=(50, 6)) for _ in range(3)], 4)
    assert A.size + sum(B.size for B in Bs) == xkv.memory_floats(50, 3, 4, 6)[0]


def test_full_rank_reconstructs_exactly():
    Xs = [rng(1).normal(size=(40, 8)) for _ in range(3)]
    A, Bs = xkv.clf(Xs, 24)
    for X, B in zip(Xs, Bs):
        np.testing.assert_allclose(xkv.reconstruct(A, B), X, rtol=0, atol=1e-12)


def test_shared_structure_is_captured_at_its_rank():
    # X_l = Z M_l: the window's concatenation has rank k whatever W is, so a
    # rank-k factorisation is exact; stacking the layers vertically instead
    # would need rank W * k
    g = rng(2)
    Z = g.normal(size=(60, 3))
    Xs = [Z @ g.normal(size=(3, 10)) for _ in range(4)]
    A, Bs = xkv.clf(Xs, 3)
    assert A.shape == (60, 3)
    for X, B in zip(Xs, Bs):
        np.testing.assert_allclose(xkv.reconstruct(A, B), X, rtol=0, atol=1e-10)


def test_rank_one_closed_form():
    # X = [x | y] with one column per layer: the best rank-1 approximation is
    # the projection on the top eigenvector of the 2x2 Gram [[a, b], [b, c]]
    x = np.array([[1.0], [2.0], [0.0]])
    y = np.array([[2.0], [1.0], [1.0]])
    a, b, c = 5.0, 4.0, 6.0
    lam = (a + c) / 2 + math.sqrt(((a - c) / 2) ** 2 + b * b)
    v = np.array([b, lam - a])
    v /= np.linalg.norm(v)
    X = np.hstack([x, y])
    best = X @ np.outer(v, v)
    A, (B1, B2) = xkv.clf([x, y], 1)
    np.testing.assert_allclose(np.hstack([A @ B1, A @ B2]), best, rtol=0, atol=1e-12)
    err2 = np.linalg.norm(X - best) ** 2
    assert err2 == pytest.approx(a + c - lam, rel=1e-12)       # trace minus the top eigenvalue


def test_no_other_subspace_does_better():
    g = rng(3)
    Xs = [g.normal(size=(80, 6)) @ np.diag(np.linspace(3, 0.2, 6)) for _ in range(2)]
    X = np.hstack(Xs)
    A, Bs = xkv.clf(Xs, 4)
    err = np.linalg.norm(X - np.hstack([A @ B for B in Bs]))
    for s in range(50):
        Q, _ = np.linalg.qr(rng(100 + s).normal(size=(12, 4)))
        assert err <= np.linalg.norm(X - X @ Q @ Q.T) + 1e-12


def test_landmarks_hand_values_and_partial_chunk():
    A = np.arange(10, dtype=float).reshape(5, 2)          # rows (0,1) (2,3) (4,5) (6,7) (8,9)
    L = xkv.landmarks(A, 2)
    np.testing.assert_array_equal(L, [[1, 2], [5, 6], [8, 9]])


def test_chunk_scores_equal_mean_reconstructed_keys():
    g = rng(4)
    A = g.normal(size=(23, 5))
    B = g.normal(size=(5, 7))
    q = g.normal(size=(3, 7))
    sc = xkv.chunk_scores(q, B, xkv.landmarks(A, 4))
    K = A @ B
    for c in range(6):
        rows = K[4 * c:min(23, 4 * c + 4)]
        want = max(sum(q[h] @ rows[i] for i in range(len(rows))) / len(rows) for h in range(3))
        assert sc[c] == pytest.approx(want, rel=1e-12, abs=1e-12)


def test_select_chunks_order_and_ties():
    s = np.array([0.5, 2.0, 2.0, -1.0, 2.0, 0.5])
    assert xkv.select_chunks(s, 2).tolist() == [1, 2]       # ties to the lower chunk
    assert xkv.select_chunks(s, 4).tolist() == [0, 1, 2, 4]
    assert xkv.select_chunks(s, 10).tolist() == [0, 1, 2, 3, 4, 5]
    assert xkv.selected_rows([1, 3], 4, 14).tolist() == [4, 5, 6, 7, 12, 13]


def test_sr_with_every_chunk_is_attention_over_reconstructed_rows():
    g = rng(5)
    Ks = [g.normal(size=(37, 16)) for _ in range(2)]
    Vs = [g.normal(size=(37, 16)) for _ in range(2)]
    AK, BKs = xkv.clf(Ks, 32)          # full rank: exact
    AV, BVs = xkv.clf(Vs, 32)
    q = g.normal(size=(4, 16))
    L = xkv.landmarks(AK, 8)
    o, lse, kept = xkv.sr_attention(q, AK, AV, BKs[1], BVs[1], L, 8, 99)
    assert kept.tolist() == [0, 1, 2, 3, 4]
    o2, lse2 = oracle.attention(q, Ks[1], Vs[1])
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


def test_sr_attends_exactly_the_selected_chunks():
    g = rng(6)
    AK, AV = g.normal(size=(64, 6)), g.normal(size=(64, 6))
    BK, BV = g.normal(size=(6, 8)), g.normal(size=(6, 8))
    q = g.normal(size=(2, 8))
    L = xkv.landmarks(AK, 8)
    o, lse, kept = xkv.sr_attention(q, AK, AV, BK, BV, L, 8, 3)
    sc = xkv.chunk_scores(q, BK, L)
    assert len(kept) == 3 and set(kept) == set(np.argsort(-sc)[:3])
    rows = xkv.selected_rows(kept, 8, 64)
    o2, lse2 = oracle.attention(q, AK[rows] @ BK, AV[rows] @ BV)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)


def test_merge_equals_attention_over_the_union():
    g = rng(7)
    K, V = g.normal(size=(30, 8)), g.normal(size=(30, 8))
    q = g.normal(size=(3, 8))
    o1, l1 = oracle.attention(q, K[:11], V[:11])
    o2, l2 = oracle.attention(q, K[11:], V[11:])
    o, lse = xkv.merge_attention(o1, l1, o2, l2)
    o3, l3 = oracle.attention(q, K, V)
    np.testing.assert_allclose(o, o3, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l3, rtol=0, atol=1e-12)
    # an empty part (lse = -inf) leaves the other unchanged
    o4, l4 = xkv.merge_attention(o1, l1, np.zeros_like(o1), np.full(3, -np.inf))
    np.testing.assert_allclose(o4, o1, rtol=0, atol=0)
    np.testing.assert_allclose(l4, l1, rtol=0, atol=0)

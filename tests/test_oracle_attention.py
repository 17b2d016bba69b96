"""Pins for the oracle's softmax decode attention and sharing map."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle


def _brute_attention(q, K, V, scale):
    """Pure-Python softmax attention of one query row (tiny inputs only)."""
    logits = [scale * sum(qa * ka for qa, ka in zip(q, k)) for k in K]
    m = max(logits)
    w = [math.exp(s - m) for s in logits]
    z = math.fsum(w)
    o = [math.fsum(wi * v[c] for wi, v in zip(w, V)) / z for c in range(len(V[0]))]
    return o, m + math.log(z)


def test_two_row_closed_form():
    # logits ln 3 and 0 give weights 3/4 and 1/4; lse = ln 4.
    d = 128
    c = 0.5
    q = np.zeros((1, d)); q[0, 5] = math.log(3.0) * math.sqrt(d) / c
    K = np.zeros((2, d)); K[0, 5] = c
    V = np.zeros((2, d)); V[0] = np.arange(d); V[1] = -2.0 * np.arange(d) + 1.0
    o, lse = oracle.attention(q, K, V)
    assert np.allclose(o[0], 0.75 * V[0] + 0.25 * V[1], rtol=1e-14, atol=1e-12)
    assert lse[0] == pytest.approx(math.log(4.0), rel=1e-14)


def test_single_row_and_equal_logits():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((3, 128))
    K = rng.standard_normal((1, 128))
    V = rng.standard_normal((1, 128))
    o, lse = oracle.attention(q, K, V)
    assert np.allclose(o, np.repeat(V, 3, axis=0), rtol=0, atol=1e-14)
    assert np.allclose(lse, q @ K[0] / math.sqrt(128), rtol=1e-14)
    K = rng.standard_normal((37, 128))
    V = rng.standard_normal((37, 128))
    o, lse = oracle.attention(np.zeros((2, 128)), K, V)
    assert np.allclose(o, V.mean(axis=0), atol=1e-14)
    assert np.allclose(lse, math.log(37), rtol=1e-14)


@pytest.mark.parametrize("T,d", [(1, 4), (5, 4), (16, 4), (9, 128)])
def test_brute_force_small(T, d):
    rng = np.random.default_rng(T * 1000 + d)
    q = rng.standard_normal((3, d))
    K = rng.standard_normal((T, d)) * 2
    V = rng.standard_normal((T, d))
    scale = 1 / math.sqrt(d)
    o, lse = oracle.attention(q, K, V)
    for r in range(3):
        ob, lb = _brute_attention(q[r].tolist(), K.tolist(), V.tolist(), scale)
        assert np.allclose(o[r], ob, rtol=1e-12, atol=1e-13)
        assert lse[r] == pytest.approx(lb, rel=1e-13)


def test_convex_hull_and_row_permutation():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 128)) * 3
    K = rng.standard_normal((300, 128))
    V = rng.standard_normal((300, 128))
    o, lse = oracle.attention(q, K, V)
    assert np.all(o <= V.max(axis=0) + 1e-12) and np.all(o >= V.min(axis=0) - 1e-12)
    perm = rng.permutation(300)
    o2, lse2 = oracle.attention(q, K[perm], V[perm])
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, lse2, rtol=1e-13)


def test_gqa_contiguous_groups():
    # KV head j holds constant value rows j + 1; head h must read head h // g.
    nb, hq, hkv, d, T = 2, 8, 2, 16, 7
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, nb, hq, d))
    K = rng.standard_normal((1, nb, hkv, T, d))
    V = np.zeros((1, nb, hkv, T, d))
    for j in range(hkv):
        V[0, :, j] = j + 1.0
    out, _ = oracle.decode_attention(q, K, V, [0], hkv, T)
    g = hq // hkv
    for h in range(hq):
        assert np.allclose(out[0, :, h], h // g + 1.0, atol=1e-14)


def test_share_map_exhaustive_small():
    for L in range(1, 9):
        for r in range(0, L):
            for rest in itertools.combinations(range(1, L), r):
                S = [0, *rest]
                src, slot = oracle.share_map(L, S)
                for layer in range(L):
                    s = src[layer]
                    assert s in S and s <= layer and S[slot[layer]] == s
                    assert not any(s < x <= layer for x in S)
                for k, s in enumerate(S):
                    assert src[s] == s and slot[s] == k


@pytest.mark.parametrize("bad", [[1, 2], [0, 0], [0, 3, 2], [0, 9], []])
def test_share_map_rejects_bad_sets(bad):
    with pytest.raises(ValueError):
        oracle.share_map(8, bad)


def test_all_leaders_is_plain_attention():
    rng = np.random.default_rng(11)
    L, nb, hq, hkv, d, T = 3, 1, 4, 2, 8, 10
    K = rng.standard_normal((L, nb, hkv, T, d))
    V = rng.standard_normal((L, nb, hkv, T, d))
    q = rng.standard_normal((L, nb, hq, d))
    _, slot = oracle.share_map(L, list(range(L)))
    out, lse = oracle.decode_attention(q, K, V, slot, hkv, T)
    for layer in range(L):
        for b in range(nb):
            for h in range(hq):
                ob, lb = _brute_attention(q[layer, b, h].tolist(),
                                          K[layer, b, h // 2].tolist(),
                                          V[layer, b, h // 2].tolist(), 1 / math.sqrt(d))
                assert np.allclose(out[layer, b, h], ob, rtol=1e-12, atol=1e-13)


def test_page_memory_figures():
    # Qwen3-8B shape, 32K context, one leader every 4 layers (bf16 assumed).
    path = os.path.join(os.path.dirname(__file__), "golden", "rcla_memory.json")
    g = json.load(open(path))
    L, hkv, d, T, elem = 36, 8, 128, 32768, 2
    _, slot = oracle.share_map(L, list(range(0, L, g["share_every_n_layers"])))
    n_slots = len(set(slot.tolist()))
    full = L * hkv * d * 2 * elem * T / 2**30
    shared = n_slots * hkv * d * 2 * elem * T / 2**30
    assert full / shared == g["stated_reduction"]
    assert abs(full - g["kv_cache_gb_full"]) / g["kv_cache_gb_full"] < 0.03
    assert abs(shared - g["kv_cache_gb_shared"]) / g["kv_cache_gb_shared"] < 0.03
    assert abs((full - shared) - g["peak_memory_saved_gb"]) / g["peak_memory_saved_gb"] < 0.05

"""Pins for the oracle's VASE selection, compaction and schedule."""
import itertools
import math

import numpy as np
import pytest
from scipy import stats

import oracle


def _rand_slab(T, seed, d=128):
    rng = np.random.default_rng(seed)
    score = rng.gamma(0.3, 1.0, size=T)
    V = rng.standard_normal((T, d))
    V[rng.choice(T, max(1, T // 100), replace=False)] *= 20
    return score, oracle.value_range(V), V


@pytest.mark.parametrize("T,K,B,Nv", [(1024, 256, 32, 16), (300, 100, 10, 0), (300, 100, 0, 100),
                                      (500, 64, 64, 64), (200, 150, 60, 5)])
def test_select_invariants(T, K, B, Nv):
    score, vr, _ = _rand_slab(T, T + K)
    d = oracle.select_detail(score, vr, T, K, B, Nv, seed=5, layer_id=3, batch=1, kv_head=2)
    kept = d["kept"]
    assert len(kept) == min(T, K + B)
    assert np.all(np.diff(kept) > 0) and kept[0] >= 0 and kept[-1] < T
    if T > K + B:
        assert set(range(T - B, T)) <= set(kept.tolist())
        cand = np.arange(T - B)
        r32 = vr.astype(np.float32)
        order = np.lexsort((cand, -r32[cand].astype(np.float64)))
        assert set(cand[order[:Nv]].tolist()) <= set(kept.tolist())
        assert len(d["sampled"]) == K - Nv


def test_select_keeps_everything_when_within_budget():
    score, vr, _ = _rand_slab(288, 1)
    assert np.array_equal(oracle.select(score, vr, 288, 256, 32, 16, 0, 0, 0, 0), np.arange(288))
    assert np.array_equal(oracle.select(score, vr, 100, 256, 32, 16, 0, 0, 0, 0), np.arange(100))


def test_nv_equal_k_is_deterministic_top_k_by_range():
    score, vr, _ = _rand_slab(700, 2)
    vr[10] = vr[11] = vr[12] = vr.max() + 1.0          # a three-way tie
    K, B = 90, 20
    cand = np.arange(700 - B)
    top = cand[np.lexsort((cand, -vr[cand].astype(np.float32).astype(np.float64)))][:K]
    want = np.sort(np.concatenate([top, np.arange(700 - B, 700)]))
    for seed in range(5):
        got = oracle.select(score, vr, 700, K, B, K, seed, 0, 0, 0)
        assert np.array_equal(got, want)


def test_zero_score_rows_only_fill_leftover_budget():
    T, K, B = 400, 120, 0
    score = np.zeros(T)
    score[:50] = 1.0                                   # only 50 positive weights
    vr = np.zeros(T)
    kept = oracle.select(score, vr, T, K, B, 0, 9, 0, 0, 0)
    assert set(range(50)) <= set(kept.tolist())
    assert np.array_equal(kept[50:], np.arange(50, 120))  # infinite keys: lowest rows


def test_uniform_weights_give_uniform_subsets():
    T, K = 40, 8
    counts = np.zeros(T)
    n = 4000
    for seed in range(n):
        kept = oracle.select(np.ones(T), np.zeros(T), T, K, 0, 0, seed, 1, 0, 0)
        counts[kept] += 1
    p = K / T
    sigma = math.sqrt(n * p * (1 - p))
    assert np.all(np.abs(counts - n * p) < 4.5 * sigma)


def test_exact_eight_token_law():
    """Successive weighted sampling without replacement, k = 3 of 8 tokens.

    Ordered triples (a, b, c) have probability
    w_a / W * w_b / (W - w_a) * w_c / (W - w_a - w_b); summing gives the
    inclusion probability of each token and of each 3-subset."""
    w = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 9.0])
    W = w.sum()
    pi = np.zeros(8)
    psub = {}
    for a, b, c in itertools.permutations(range(8), 3):
        pr = w[a] / W * w[b] / (W - w[a]) * w[c] / (W - w[a] - w[b])
        pi[[a, b, c]] += pr
        key = tuple(sorted((a, b, c)))
        psub[key] = psub.get(key, 0.0) + pr
    assert len(psub) == 56 and pi.sum() == pytest.approx(3.0)
    n = 10000
    freq = np.zeros(8)
    sub_counts = {k: 0 for k in psub}
    for seed in range(n):
        kept = oracle.select(w, np.zeros(8), 8, 3, 0, 0, seed, 2, 0, 1)
        freq[kept] += 1
        sub_counts[tuple(kept.tolist())] += 1
    sigma = np.sqrt(n * pi * (1 - pi))
    assert np.all(np.abs(freq - n * pi) <= 4 * sigma)
    obs = np.array([sub_counts[k] for k in psub])
    exp = np.array([psub[k] for k in psub]) * n
    chi2 = ((obs - exp) ** 2 / exp).sum()
    assert stats.chi2.sf(chi2, 55) > 1e-3


def test_select_rejects_bad_budget():
    with pytest.raises(ValueError):
        oracle.select(np.ones(10), np.ones(10), 10, 2, 0, 3, 0, 0, 0, 0)


def test_compact_gathers_rows_and_restricts_attention():
    rng = np.random.default_rng(6)
    T, d = 120, 128
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    kept = np.sort(rng.choice(T, 50, replace=False))
    K2, V2 = oracle.compact(K, V, kept)
    assert np.array_equal(K2, K[kept]) and np.array_equal(V2, V[kept])
    q = rng.standard_normal((2, d))
    o2, _ = oracle.attention(q, K2, V2)
    # attention with the evicted rows masked out, by brute force
    for r in range(2):
        logits = {t: float(q[r] @ K[t]) / math.sqrt(d) for t in kept}
        m = max(logits.values())
        e = {t: math.exp(s - m) for t, s in logits.items()}
        z = math.fsum(e.values())
        o = sum(e[t] * V[t] for t in kept) / z
        assert np.allclose(o2[r], o, rtol=1e-12, atol=1e-13)


def test_schedule_eviction_count_and_bounds():
    # Qwen3-4B-shaped VASE run: 16384 steps from empty, K=4096, B=128, P=128.
    K, B, P = 4096, 128, 128
    t, n, lo, hi = 0, 0, None, 0
    for s in range(16384):
        t += 1
        hi = max(hi, t)
        if oracle.eviction_due(s, P, t, K, B):
            t = K + B
            n += 1
            lo = t if lo is None else min(lo, t)
    assert n == 95 and hi == K + B + P and lo == K + B


def test_run_decode_small_trajectory_properties():
    rng = np.random.default_rng(12)
    L, leaders, nb, hq, hkv, d, T0, steps = 4, [0, 2], 1, 4, 2, 16, 40, 8
    K0 = rng.standard_normal((2, nb, hkv, T0, d))
    V0 = rng.standard_normal((2, nb, hkv, T0, d))
    q = rng.standard_normal((steps, L, nb, hq, d))
    kn = rng.standard_normal((steps, 2, nb, hkv, d))
    vn = rng.standard_normal((steps, 2, nb, hkv, d))
    ev = dict(K=20, B=4, N_v=2, period=4, w=4, seed=3)
    outs, Kc, Vc, t_len, rec = oracle.run_decode(L, leaders, K0, V0, T0, q, kn, vn, ev)
    assert outs.shape == (steps, L, nb, hq, d)
    # evictions after steps 3 and 7 (44 -> 24, 28 -> 24 rows)
    assert t_len == 20 + 4 and len(rec) == 2 * 2 * nb * hkv
    # follower layers 1 and 3 read their leader's cache: at step 0 the
    # output for layer 1 equals attention of its queries over slot 0
    o, _ = oracle.attention(q[0, 1, 0, 0:2], np.concatenate([K0[0, 0, 0], kn[0, 0, 0, 0][None]]),
                            np.concatenate([V0[0, 0, 0], vn[0, 0, 0, 0][None]]))
    assert np.allclose(outs[0, 1, 0, 0:2], o, rtol=1e-13)

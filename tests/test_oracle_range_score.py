"""Pins for the oracle's value range and observation-window score."""
import math

import numpy as np
import pytest
import torch

import oracle


def test_range_hand_values_and_invariances():
    V = np.array([[1.0, -2.0, 3.0, 0.5], [0.0, 0.0, 0.0, 0.0], [-1.0, -4.0, -2.5, -3.0]])
    assert np.array_equal(oracle.value_range(V), [5.0, 0.0, 3.0])
    rng = np.random.default_rng(2)
    V = rng.standard_normal((50, 128))
    r = oracle.value_range(V)
    assert np.allclose(oracle.value_range(V + 7.25), r, rtol=1e-12)
    assert np.allclose(oracle.value_range(-2 * V), 2 * r, rtol=1e-12)
    assert np.array_equal(oracle.value_range(V[:, rng.permutation(128)]), r)


def test_range_of_bf16_rows_rounds_like_float32():
    # For bfloat16 inputs the float64 range is exact; rounding it once to
    # float32 must equal float32 max minus float32 min (one IEEE rounding).
    g = torch.Generator().manual_seed(4)
    V = torch.randn(4096, 128, generator=g)
    V[::97] *= 20
    V = V.to(torch.bfloat16)
    ref = (V.float().amax(-1) - V.float().amin(-1)).numpy()
    got = oracle.value_range(V.double().numpy()).astype(np.float32)
    assert np.array_equal(got, ref)


def _brute_score(q_obs, K, t_len, scale):
    w, g, d = len(q_obs), len(q_obs[0]), len(q_obs[0][0])
    score = [0.0] * t_len
    for i in range(w):
        vis = t_len - w + i + 1
        for h in range(g):
            logits = [scale * sum(a * b for a, b in zip(q_obs[i][h], K[t])) for t in range(vis)]
            m = max(logits)
            e = [math.exp(s - m) for s in logits]
            z = math.fsum(e)
            for t in range(vis):
                score[t] += e[t] / z
    return score


def test_score_uniform_causal_closed_form():
    # All-zero queries give uniform rows; row i sees t_len - w + i + 1 rows.
    w, g, d, T = 4, 3, 128, 9
    K = np.random.default_rng(0).standard_normal((T, d))
    sc = oracle.window_score(np.zeros((w, g, d)), K, T)
    want = np.zeros(T)
    for i in range(w):
        vis = T - w + i + 1
        want[:vis] += g / vis
    assert np.allclose(sc, want, rtol=1e-14)
    # w = 2, T = 3, g = 1: [1/2 + 1/3, 1/2 + 1/3, 1/3]
    sc = oracle.window_score(np.zeros((2, 1, 128)), K[:3], 3)
    assert np.allclose(sc, [5 / 6, 5 / 6, 1 / 3], rtol=1e-14)


@pytest.mark.parametrize("T,w,g", [(6, 3, 2), (16, 4, 1), (12, 12, 2)])
def test_score_brute_force_and_row_sums(T, w, g):
    rng = np.random.default_rng(T + w + g)
    q = rng.standard_normal((w, g, 8)) * 2
    K = rng.standard_normal((T, 8))
    sc = oracle.window_score(q, K, T)
    bf = _brute_score(q.tolist(), K.tolist(), T, 1 / math.sqrt(8))
    assert np.allclose(sc, bf, rtol=1e-12, atol=1e-14)
    assert sc.sum() == pytest.approx(g * w, rel=1e-13)


def test_score_single_row_equals_attention_weights():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 1, 128))
    K = rng.standard_normal((40, 128))
    sc = oracle.window_score(q, K, 40)
    _, lse = oracle.attention(q[0], K, K)
    assert np.allclose(sc, np.exp(q[0, 0] @ K.T / math.sqrt(128) - lse[0]), rtol=1e-12)


def test_score_needs_window_rows():
    with pytest.raises(ValueError):
        oracle.window_score(np.zeros((4, 1, 8)), np.zeros((3, 8)), 3)

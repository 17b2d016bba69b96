"""Pins of the range-protected quantization oracle (oracle/quant.py): hand
values, the rounding bound, exact scalings, the protection rule and the
page's claim that large-range value rows dominate the per-token error."""
import numpy as np
import pytest

import oracle
from oracle import quant


def rng(s):
    return np.random.default_rng(s)


def bf16(x):
    """Round float64 values to bfloat16 (nearest even), back to float64."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def test_hand_values():
    X = np.array([[127.0, -63.5, 0.375, -0.625, 2.5, 3.5, -127.0, 0.5]])
    codes, scale = quant.quantize_rows(X)
    assert scale[0] == 1.0
    # round half to even: -63.5 -> -64, 2.5 -> 2, 3.5 -> 4, 0.5 -> 0
    assert codes[0].tolist() == [127, -64, 0, -1, 2, 4, -127, 0]


def test_zero_row_and_scale():
    X = np.zeros((2, 8))
    X[1, 3] = -2.5
    codes, scale = quant.quantize_rows(X)
    assert scale[0] == 0 and not codes[0].any()
    assert scale[1] == np.float32(2.5 / 127) and codes[1, 3] == -127


def test_rounding_bound_and_extremes():
    X = bf16(rng(0).normal(size=(500, 128)) * rng(1).uniform(0.01, 30, size=(500, 1)))
    codes, scale = quant.quantize_rows(X)
    err = np.abs(X - quant.dequantize_rows(codes, scale))
    assert np.all(err <= scale[:, None].astype(np.float64) * 0.50001)
    # the element of largest magnitude maps to +-127
    idx = np.abs(X).argmax(axis=1)
    assert np.all(np.abs(codes[np.arange(500), idx]) == 127)


def test_power_of_two_scaling_and_sign():
    X = bf16(rng(2).normal(size=(50, 64)))
    c1, s1 = quant.quantize_rows(X)
    c2, s2 = quant.quantize_rows(X * 8.0)
    c3, s3 = quant.quantize_rows(-X)
    assert np.array_equal(c1, c2) and np.array_equal(s2, s1 * np.float32(8))
    assert np.array_equal(c3, -c1) and np.array_equal(s3, s1)


def test_protection_picks_largest_ranges_lower_row_on_ties():
    V = np.zeros((10, 4))
    V[:, 0] = [1, 5, 2, 5, 3, 0, 9, 5, 1, 1]
    assert quant.protected_rows(V, 3).tolist() == [1, 3, 6]      # 9, then 5, 5 (rows 1, 3)
    assert quant.protected_rows(V, 0).tolist() == []
    assert quant.protected_rows(V, 50).tolist() == list(range(10))


def test_all_rows_protected_is_plain_attention():
    g = rng(3)
    K, V = bf16(g.normal(size=(40, 16))), bf16(g.normal(size=(40, 16)))
    q = bf16(g.normal(size=(3, 16)))
    o1, l1 = quant.quantized_attention(q, K, V, 40)
    o2, l2 = oracle.attention(q, K, V)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_exactly_representable_rows_reconstruct_exactly():
    g = rng(4)
    K = g.integers(-127, 128, size=(30, 8)).astype(np.float64)
    V = g.integers(-127, 128, size=(30, 8)).astype(np.float64)
    K[:, 0], V[:, 0] = 127, -127           # amax 127 in every row: scale 1
    Kh, Vh, _ = quant.reconstruct(K, V, 0)
    assert np.array_equal(Kh, K) and np.array_equal(Vh, V)
    q = g.normal(size=(2, 8))
    o1, _ = quant.quantized_attention(q, K, V, 0)
    o2, _ = oracle.attention(q, K, V)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)


def test_large_range_rows_dominate_the_error():
    # one value row with 20x the range of the others: without protection its
    # per-token step is ~20x larger and it holds the largest errors; keeping
    # it in bf16 brings the worst error down to the other rows' level.
    g = rng(5)
    T, d = 200, 128
    V = bf16(g.normal(size=(T, d)))
    V[37] = bf16(V[37] * 20)
    K = bf16(g.normal(size=(T, d)))
    Kh, Vh, prot = quant.reconstruct(K, V, 0)
    e0 = np.abs(Vh - V).max(axis=1)
    assert e0.argmax() == 37 and e0[37] > 8 * np.delete(e0, 37).max()
    Kh, Vh, prot = quant.reconstruct(K, V, 1)
    assert prot.tolist() == [37]
    e1 = np.abs(Vh - V).max(axis=1)
    assert e1[37] == 0 and e1.max() == np.delete(e0, 37).max()

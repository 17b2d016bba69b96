"""Range-protected per-token KV quantization, for the oracle (test
infrastructure).

TEST INFRASTRUCTURE ONLY: tests/, the package's smoke check and the CPU
baseline leg of bench.py are the only code that may import it.  It shares no
code with the HIP library.

The VASE summary (gist.science 2606.03928), §3 (third contribution) and §5:
value states of large range are the main source of reconstruction error
when the KV cache is quantized per token, so a mixed-precision scheme should
keep those high-magnitude states at full precision.  The pages give no
format; the reading fixed here is the plainest one:

* every cached row (one token of one KV head) is quantized on its own, its
  key row and its value row separately, symmetric int8 with one float32
  scale per row: scale = max_c |x_c| / 127 (float32 division), code_c =
  round-half-even(x_c / scale) (float32 division), clamped to [-127, 127];
  a row of zeros has scale 0 and codes 0;
* the P rows of largest value range (Range(v) = max(v) - min(v), §2.A; ties
  to the lower row) keep their bfloat16 key and value rows instead;
* the reconstruction of a quantized row is code_c * scale (exact), and
  decode attention runs on the reconstructed rows (plain softmax attention
  over all rows, protected or not).
"""
import numpy as np

from .kvc_oracle import attention, value_range

QMAX = 127


def quantize_rows(X):
    """X: [T][d] values (float64 holding bf16 numbers).  Returns codes
    (int8 [T][d]) and scales (float32 [T])."""
    X32 = np.asarray(X, dtype=np.float32)
    amax = np.abs(X32).max(axis=1)
    scale = (amax / np.float32(QMAX)).astype(np.float32)
    codes = np.zeros(X32.shape, dtype=np.int8)
    nz = scale > 0
    if nz.any():
        r = (X32[nz] / scale[nz, None]).astype(np.float32)
        codes[nz] = np.clip(np.rint(r), -QMAX, QMAX).astype(np.int8)
    return codes, scale


def dequantize_rows(codes, scale):
    return codes.astype(np.float64) * scale.astype(np.float64)[:, None]


def protected_rows(V, n_protect):
    """Rows of the P largest value ranges, ascending (ties to the lower row)."""
    r = value_range(V)
    T = len(r)
    P = min(int(n_protect), T)
    order = np.lexsort((np.arange(T), -r))
    return np.sort(order[:P])


def reconstruct(K, V, n_protect):
    """The rows decode attention sees after range-protected quantization:
    returns (K_hat, V_hat, protected index array)."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    prot = protected_rows(V, n_protect)
    ck, sk = quantize_rows(K)
    cv, sv = quantize_rows(V)
    Kh, Vh = dequantize_rows(ck, sk), dequantize_rows(cv, sv)
    Kh[prot], Vh[prot] = K[prot], V[prot]
    return Kh, Vh, prot


def quantized_attention(q, K, V, n_protect, scale=None):
    """Decode attention of the query rows q [g][d] over the reconstructed
    rows of one slab; returns (o, lse) like attention()."""
    Kh, Vh, _ = reconstruct(K, V, n_protect)
    return attention(q, Kh, Vh, scale)

"""Cross-layer factorisation and selective reconstruction, for the oracle
(test infrastructure).

TEST INFRASTRUCTURE ONLY: tests/, the package's smoke check and the CPU
baseline leg of bench.py are the only code that may import it.  It shares no
code with the HIP library.

xKV summary (gist.science 2503.18893):
* §2.2 (cross-layer factorisation): the layers are cut into windows of W
  consecutive layers; the KV caches of a window are concatenated side by
  side and a rank-r SVD of the concatenation yields one token basis A shared
  by the window and one reconstruction matrix B_l per layer, so W full
  caches (W x T x d numbers) become T x r + W x r x d numbers;
* §2.3 (selective reconstruction): at decode, landmark-based chunk selection
  picks the chunks of tokens most relevant to the current query, and only
  their rows are rebuilt from A and B_l before attention.

Readings fixed here (the page gives no more detail):
* one factorisation per (batch entry, KV head, window), keys and values
  separately: X = [X_1 | ... | X_W] (T x W*d), truncated SVD
  X ~ U_r S_r V_r^T, A = U_r S_r (T x r), [B_1 | ... | B_W] = V_r^T (each
  B_l r x d), reconstruction X_l ~ A B_l;
* chunks are c consecutive rows (the last one may be shorter); the landmark
  of a chunk is the mean of its rows of A (so that the landmark's key,
  mean(A) B_l, is the mean of the chunk's reconstructed keys);
* chunk score for the g query heads of one KV head: the maximum over the
  heads of q_h . (landmark key); the n_select chunks of largest score are
  kept (ties to the lower chunk), all of them when there are fewer;
* attention runs over the reconstructed rows of the kept chunks, in row
  order; rows appended after the factorisation (decode) are attended
  uncompressed and the two parts merge exactly (log-sum-exp).
"""
import math

import numpy as np

from .kvc_oracle import attention


def clf(Xs, rank):
    """Cross-layer factorisation of one window.

    Xs: list of W arrays [T][d] (the window's layers, one KV head of one
    batch entry).  Returns (A [T][r], [B_1, ..., B_W] each [r][d])."""
    X = np.concatenate([np.asarray(x, dtype=np.float64) for x in Xs], axis=1)
    U, s, Vt = np.linalg.svd(X, full_matrices=False)
    r = min(rank, len(s))
    A = U[:, :r] * s[:r]
    d = np.asarray(Xs[0]).shape[1]
    Bs = [Vt[:r, l * d:(l + 1) * d] for l in range(len(Xs))]
    return A, Bs


def reconstruct(A, B):
    """Rows of one layer rebuilt from the shared basis: A B_l."""
    return np.asarray(A, dtype=np.float64) @ np.asarray(B, dtype=np.float64)


def memory_floats(T, W, r, d):
    """Numbers stored for one window: the shared T x r basis and W r x d
    matrices, against W x T x d for the full caches."""
    return T * r + W * r * d, W * T * d


def landmarks(A, chunk):
    """Mean of each chunk's rows of A: [ceil(T / chunk)][r]."""
    A = np.asarray(A, dtype=np.float64)
    T = A.shape[0]
    n = (T + chunk - 1) // chunk
    return np.stack([A[i * chunk:min(T, (i + 1) * chunk)].mean(axis=0) for i in range(n)])


def chunk_scores(q, B, L):
    """Score of every chunk for the query rows q [g][d] of one KV head:
    max over the heads of q_h . (L_c B_l)."""
    keys = np.asarray(L, dtype=np.float64) @ np.asarray(B, dtype=np.float64)   # [n][d]
    return (np.asarray(q, dtype=np.float64) @ keys.T).max(axis=0)


def select_chunks(scores, n_select):
    """Ascending indices of the n_select largest scores (ties to the lower
    chunk); every chunk when there are at most n_select."""
    scores = np.asarray(scores, dtype=np.float64)
    n = len(scores)
    k = min(n_select, n)
    order = np.lexsort((np.arange(n), -scores))
    return np.sort(order[:k])


def selected_rows(chunks, chunk, T):
    return np.concatenate([np.arange(c * chunk, min(T, (c + 1) * chunk)) for c in chunks]) \
        if len(chunks) else np.zeros(0, dtype=np.int64)


def sr_attention(q, AK, AV, BK, BV, L, chunk, n_select, scale=None):
    """Selective reconstruction for the query rows q [g][d] of one KV head
    and one layer: select chunks by their landmarks, rebuild their key and
    value rows, attend.  Returns (o [g][d], lse [g], kept chunk indices)."""
    T = np.asarray(AK).shape[0]
    sc = chunk_scores(q, BK, L)
    kept = select_chunks(sc, n_select)
    rows = selected_rows(kept, chunk, T)
    Kh = reconstruct(np.asarray(AK, dtype=np.float64)[rows], BK)
    Vh = reconstruct(np.asarray(AV, dtype=np.float64)[rows], BV)
    o, lse = attention(q, Kh, Vh, scale)
    return o, lse, kept


def merge_attention(o1, lse1, o2, lse2):
    """Attention over the union of two disjoint row sets from the two parts'
    outputs and log-normalisers (an empty part has lse = -inf)."""
    o1, o2 = np.asarray(o1, dtype=np.float64), np.asarray(o2, dtype=np.float64)
    lse1, lse2 = np.asarray(lse1, dtype=np.float64), np.asarray(lse2, dtype=np.float64)
    m = np.maximum(lse1, lse2)
    w1 = np.where(np.isneginf(lse1), 0.0, np.exp(lse1 - m))
    w2 = np.where(np.isneginf(lse2), 0.0, np.exp(lse2 - m))
    z = w1 + w2
    o = (o1 * w1[..., None] + o2 * w2[..., None]) / z[..., None]
    return o, m + np.log(z)

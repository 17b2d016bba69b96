"""VASE-DKV token scores for the oracle (test infrastructure).

TEST INFRASTRUCTURE ONLY: tests/, the package's smoke check and the CPU
baseline leg of bench.py are the only code that may import it.  It shares no
code with the HIP library.

The VASE summary (gist.science 2606.03928, §2.B) describes VASE-DKV only as
CurDKV's scoring, whose token scores are leverage scores from a CUR matrix
decomposition, with a Gaussian projection matrix G drawn afresh at every
eviction pass so that no token keeps a low score by construction.  The pages
give no formula, so this module fixes the plainest one that fits those words:

* the matrix whose rows are scored is A = [K | V], the key row and the value
  row of each cached token side by side (T x 2d);
* the Gaussian projection sketches it, Y = A G with G of shape (2d, r) and
  independent N(0, 1) entries;
* the score of token t is the statistical leverage of row t of Y,
  l_t = y_t (Y^T Y)^+ y_t^T, i.e. the squared norm of row t of an orthonormal
  basis of the column space of Y.  This is the standard sketched
  approximation of rank-r leverage scores (a Gaussian range finder followed by
  exact leverage of the sketch); with r >= rank(A) it equals the leverage of
  A itself, and sum_t l_t = rank(Y).
* (Y^T Y)^+ is taken through a Cholesky factorisation that drops every
  direction whose pivot is at most 1e-12 of the Gram matrix's trace (rank
  deficiency: fewer independent rows than r).

The sampling then runs exactly as for the window scores (weights l_t, the
same exponential keys, the same N_v range protection and recent buffer).

G is an input.  gaussian_bf16 defines the generator the library exports for
it: Box-Muller (1958) on Philox4x32-10 words, element 2p and 2p+1 from the
words x0, x1 at counter (p, c1, c2, 0) under the seed's key,
    u1 = (x0 + 1) / 2^32 in (0, 1],  u2 = x1 / 2^32 in [0, 1),
    z_2p = sqrt(-2 ln u1) cos(2 pi u2),  z_2p+1 = sqrt(-2 ln u1) sin(2 pi u2),
evaluated in float64, rounded to float32 and then to bfloat16 (both round to
nearest even).
"""
import numpy as np

from .philox import philox4x32_10, seed_key

DROP_REL = 1e-12


# --------------------------------------------------------------------------
# Gaussian projection entries
# --------------------------------------------------------------------------
def bf16_round_bits(x32):
    """float32 array -> bfloat16 bit patterns (uint16), round to nearest even
    on the 16 dropped bits (finite inputs)."""
    b = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    return ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def box_muller(x0, x1):
    """Two standard normals per pair of 32-bit words, float64."""
    u1 = (np.asarray(x0, dtype=np.float64) + 1.0) / 4294967296.0
    u2 = np.asarray(x1, dtype=np.float64) / 4294967296.0
    rad = np.sqrt(-2.0 * np.log(u1))
    th = 2.0 * np.pi * u2
    return rad * np.cos(th), rad * np.sin(th)


def gaussian_bf16(n, seed, c1, c2):
    """n N(0, 1) draws as bfloat16 bit patterns (uint16[n])."""
    pairs = (n + 1) // 2
    p = np.arange(pairs, dtype=np.uint64)
    k0, k1 = seed_key(seed)
    x0, x1, _, _ = philox4x32_10(p, np.uint64(c1), np.uint64(c2), np.uint64(0),
                                 np.uint64(k0), np.uint64(k1))
    z0, z1 = box_muller(x0, x1)
    z = np.empty(2 * pairs, dtype=np.float64)
    z[0::2], z[1::2] = z0, z1
    return bf16_round_bits(z[:n].astype(np.float32))


# --------------------------------------------------------------------------
# Leverage of the sketched rows
# --------------------------------------------------------------------------
def sketch(K, V, G):
    """Y = [K | V] G, float64.  K, V: [T][d]; G: [2d][r]."""
    A = np.concatenate([np.asarray(K, np.float64), np.asarray(V, np.float64)], axis=1)
    return A @ np.asarray(G, np.float64)


def cholesky_drop(M, rel=DROP_REL):
    """Upper-triangular R with R^T R = M on the kept directions, plus the
    kept mask.  A direction is dropped (its row of R is zero) when its pivot
    is <= rel * trace(M)."""
    M = np.asarray(M, np.float64)
    r = M.shape[0]
    R = np.zeros((r, r))
    keep = np.zeros(r, dtype=bool)
    floor = rel * max(np.trace(M), 0.0)
    for j in range(r):
        s = M[j, j] - np.dot(R[:j, j], R[:j, j])
        if not s > floor:
            continue
        keep[j] = True
        R[j, j] = np.sqrt(s)
        for i in range(j + 1, r):
            R[j, i] = (M[j, i] - np.dot(R[:j, j], R[:j, i])) / R[j, j]
    return R, keep


def leverage_of_sketch(Y, rel=DROP_REL):
    """l_t = ||y_t[kept] R_kk^{-1}||^2 for the rows of Y."""
    Y = np.asarray(Y, np.float64)
    R, keep = cholesky_drop(Y.T @ Y, rel)
    if not keep.any():
        return np.zeros(Y.shape[0])
    Rk = R[np.ix_(keep, keep)]
    Z = np.linalg.solve(Rk.T, Y[:, keep].T).T     # Z = Y_k Rk^{-1}
    return (Z * Z).sum(axis=1)


def dkv_score(K, V, G, rel=DROP_REL):
    """VASE-DKV token scores of one slab: leverage of the rows of [K | V] G."""
    return leverage_of_sketch(sketch(K, V, G), rel)

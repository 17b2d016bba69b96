"""Plain float64 CPU oracle for decode attention over a compressed KV cache.

TEST INFRASTRUCTURE ONLY.  Only tests/, the package's smoke check and the CPU
baseline leg of bench.py may import or call anything under oracle/.  The
product path never routes through this module, and this module shares no
code with the HIP library.

Everything is written from the statement of the method on three pages:

* "Stochastic KV Routing" (aitrends.kr article on R-CLA), the inference and
  implementation paragraphs: a fixed sharing set S; a layer outside S reuses
  the KV of the nearest earlier layer in S, and only layers in S store new
  KV.
* "VASE: value-aware stochastic KV-cache eviction" (gist.science 2606.03928),
  §2: periodic eviction holding a persistent budget K plus a recent buffer B;
  §2.A: Range(v) = max(v) - min(v) and the N_v tokens of largest range are
  always kept; §2.B: the rest of the budget is filled by weighted random
  sampling on attention scores derived from SnapKV's observation window.
* Decode attention itself is ordinary softmax attention of one query per
  head over the rows of the cache it reads.

Arrays are numpy; every floating-point step is float64 unless a docstring
says otherwise.  One "slab" is the [T][d] block of one (batch entry, cache
slot, KV head).  K and V are passed in logical row-major form [T][d].

Readings of points the pages leave open:
  GQA: query head h reads KV head h // g (contiguous groups).
  Scale: softmax of q.k / sqrt(d) unless a scale is given.
  S must contain layer 0; the recent buffer is the last B rows; N_v is
  drawn from the candidate rows [0, T-B); ties go to the lower row index;
  the window score sums softmax probabilities over the window rows and the
  GQA group, window row i seeing rows t <= T - w + i; sampling without
  replacement proportional to score is realised by exponential keys
  kappa_t = E_t / score_t with E_t from Philox4x32-10 word 0 at counter
  (t, kv_head, layer, batch) and key (seed low, seed high).
"""
import math

import numpy as np

from .philox import philox4x32_10, seed_key

TWO32 = 4294967296.0


# --------------------------------------------------------------------------
# O1  sharing map (Stochastic KV Routing, inference paragraph)
# --------------------------------------------------------------------------
def share_map(n_layers, leaders):
    """Nearest earlier leader for every layer.

    Layer l reads the KV of src(l) = max{s in S : s <= l}; slot(l) is the
    position of src(l) in the sorted set S.  Layer 0 must be a leader (the
    pages give no source for a layer with no earlier cached layer)."""
    leaders = [int(s) for s in leaders]
    if n_layers < 1 or not leaders:
        raise ValueError("need at least one layer and one leader")
    if leaders[0] != 0:
        raise ValueError("layer 0 must be in the sharing set")
    for a, b in zip(leaders, leaders[1:]):
        if not a < b:
            raise ValueError("leaders must be strictly increasing")
    if leaders[-1] >= n_layers:
        raise ValueError("leader out of range")
    src_layer = np.empty(n_layers, dtype=np.int32)
    src_slot = np.empty(n_layers, dtype=np.int32)
    for layer in range(n_layers):
        best = None
        for slot, s in enumerate(leaders):
            if s <= layer:
                best = (s, slot)
        src_layer[layer], src_slot[layer] = best
    return src_layer, src_slot


# --------------------------------------------------------------------------
# O2  leader append (Stochastic KV Routing, implementation paragraph)
# --------------------------------------------------------------------------
def append_row(K, V, t_len, k_new, v_new):
    """Write the new row at index t_len of a slab and return t_len + 1.

    Only leader layers call this; followers store nothing."""
    K[t_len] = k_new
    V[t_len] = v_new
    return t_len + 1


# --------------------------------------------------------------------------
# O3  softmax attention of a few query rows over one slab
# --------------------------------------------------------------------------
def attention(q, K, V, scale=None):
    """o = softmax(q K^T * scale) V and lse = log sum exp(q K^T * scale).

    q: [R][d] query rows that share this slab; K, V: [T][d]."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    d = q.shape[-1]
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    s = (q @ K.T) * scale                      # [R][T]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    z = p.sum(axis=1, keepdims=True)
    o = (p @ V) / z
    lse = (m + np.log(z))[:, 0]
    return o, lse


def decode_attention(q, K_slots, V_slots, q_slot, n_kv_heads, t_len, scale=None):
    """Grouped-query decode attention of several q-layers over leader slots.

    q: [nq][nb][Hq][d]; K_slots, V_slots: [n_slots][nb][Hkv][>=t_len][d];
    q_slot[i] is the cache slot q-layer i reads (its nearest earlier leader).
    Query head h reads KV head h // (Hq / Hkv).  Returns out [nq][nb][Hq][d]
    and lse [nq][nb][Hq]."""
    q = np.asarray(q)
    nq, nb, hq, d = q.shape
    g = hq // n_kv_heads
    out = np.zeros((nq, nb, hq, d))
    lse = np.zeros((nq, nb, hq))
    for i in range(nq):
        slot = int(q_slot[i])
        for b in range(nb):
            for j in range(n_kv_heads):
                heads = slice(j * g, (j + 1) * g)
                o, l = attention(q[i, b, heads], K_slots[slot][b][j][:t_len],
                                 V_slots[slot][b][j][:t_len], scale)
                out[i, b, heads] = o
                lse[i, b, heads] = l
    return out, lse


# --------------------------------------------------------------------------
# O4  value range (VASE §2.A)
# --------------------------------------------------------------------------
def value_range(V):
    """Range(v) = max(v) - min(v) over the channels of each value row.

    V: [T][d] -> [T] float64 (exact for bfloat16 or float32 inputs of
    similar magnitude)."""
    V = np.asarray(V, dtype=np.float64)
    return V.max(axis=-1) - V.min(axis=-1)


# --------------------------------------------------------------------------
# O5  observation-window score (VASE §2.B, SnapKV-derived)
# --------------------------------------------------------------------------
def window_score(q_obs, K, t_len, scale=None):
    """Sum of window softmax probabilities for every cached row.

    q_obs: [w][g][d], the last w decode queries of the g query heads that
    read this KV head, oldest first.  Window row i was issued when the cache
    held t_len - w + i + 1 rows, so it sees rows t <= t_len - w + i.
    score[t] = sum over heads and window rows of softmax_t(q.k_t * scale).
    Returns [t_len] float64."""
    q_obs = np.asarray(q_obs, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)[:t_len]
    w, g, d = q_obs.shape
    if t_len < w:
        raise ValueError("the window needs at least w cached rows")
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    score = np.zeros(t_len)
    for i in range(w):
        visible = t_len - w + i + 1
        s = (q_obs[i] @ K[:visible].T) * scale     # [g][visible]
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        p /= p.sum(axis=1, keepdims=True)
        score[:visible] += p.sum(axis=0)
    return score


# --------------------------------------------------------------------------
# O6  selection (VASE §2, §2.A, §2.B)
# --------------------------------------------------------------------------
def philox_word0(t, kv_head, layer_id, batch, seed):
    """Word 0 of Philox4x32-10 at counter (t, kv_head, layer_id, batch) and
    key (seed mod 2**32, seed >> 32); t may be an array."""
    k0, k1 = seed_key(seed)
    t = np.asarray(t, dtype=np.uint64)
    x, _, _, _ = philox4x32_10(t, kv_head, layer_id, batch, k0, k1)
    return x


def exp_variate(x):
    """Unit exponential variate from a 32-bit word: E = -ln((x + 1) / 2**32).

    Computed as -log1p(-m / 2**32) with m = 2**32 - 1 - x so that words near
    2**32 keep full relative accuracy."""
    x = np.asarray(x, dtype=np.float64)
    m = (TWO32 - 1.0) - x
    return -np.log1p(-m / TWO32)


def select_detail(score, vrange, t_len, budget_k, recent_b, n_v, seed,
                  layer_id, batch, kv_head):
    """VASE selection for one slab, with the quantities that decide it.

    If t_len <= K + B every row is kept.  Otherwise the last B rows are kept,
    then the N_v candidates of largest range (ties to the lower row), then
    K - N_v more rows sampled without replacement with probability
    proportional to score: exponential keys kappa_t = E_t / score_t (an
    infinite key when score_t <= 0), smallest keys first, ties to the lower
    row.  The range decision is taken on float32 ranges (the precision of
    the device path); the key decision in float64.

    Returns a dict with 'kept' (ascending int64 rows), 'protected' (the N_v
    rows), 'sampled', 'kappa' (float64 per row, inf outside the sampling
    pool), 'kappa_cut' (largest sampled key) and 'range_cut' (smallest
    protected float32 range)."""
    score = np.asarray(score, dtype=np.float64)[:t_len]
    vr32 = np.asarray(vrange, dtype=np.float64)[:t_len].astype(np.float32)
    if not (0 <= n_v <= budget_k and recent_b >= 0):
        raise ValueError("need 0 <= N_v <= K and B >= 0")
    rows = np.arange(t_len)
    out = dict(protected=np.zeros(0, np.int64), sampled=np.zeros(0, np.int64),
               kappa=np.full(t_len, np.inf), kappa_cut=None, range_cut=None)
    if t_len <= budget_k + recent_b:
        out["kept"] = rows.astype(np.int64)
        return out
    n_cand = t_len - recent_b
    cand = rows[:n_cand]
    # top-N_v by (range descending, row ascending)
    order = np.lexsort((cand, -vr32[:n_cand].astype(np.float64)))
    protected = np.sort(cand[order[:n_v]])
    pool = np.setdiff1d(cand, protected)
    # exponential keys for the sampling pool
    x = philox_word0(pool, kv_head, layer_id, batch, seed)
    e = exp_variate(x)
    sc = score[pool]
    with np.errstate(divide="ignore", invalid="ignore"):
        kappa = np.where(sc > 0, e / np.where(sc > 0, sc, 1.0), np.inf)
    n_s = budget_k - n_v
    korder = np.lexsort((pool, kappa))
    sampled = np.sort(pool[korder[:n_s]])
    kept = np.sort(np.concatenate([rows[n_cand:], protected, sampled]))
    out.update(kept=kept.astype(np.int64), protected=protected.astype(np.int64),
               sampled=sampled.astype(np.int64))
    out["kappa"][pool] = kappa
    if n_s > 0:
        out["kappa_cut"] = float(kappa[korder[n_s - 1]])
    if n_v > 0:
        out["range_cut"] = float(vr32[protected].min())
    return out


def select(score, vrange, t_len, budget_k, recent_b, n_v, seed, layer_id,
           batch, kv_head):
    """Ascending kept rows of one slab (see select_detail)."""
    return select_detail(score, vrange, t_len, budget_k, recent_b, n_v, seed,
                         layer_id, batch, kv_head)["kept"]


# --------------------------------------------------------------------------
# O7  compaction (VASE §1: evicted pairs are dropped for good)
# --------------------------------------------------------------------------
def compact(K, V, kept):
    """Gather the kept rows, in ascending order, into a new slab."""
    kept = np.asarray(kept, dtype=np.int64)
    return np.asarray(K)[kept].copy(), np.asarray(V)[kept].copy()


# --------------------------------------------------------------------------
# O8  periodic schedule (VASE §2: periodic eviction with budget K + B)
# --------------------------------------------------------------------------
def eviction_due(step, period, t_len, budget_k, recent_b):
    """After decode step `step` (0-based) an eviction pass runs when
    (step + 1) is a multiple of the period and the cache exceeds K + B."""
    return (step + 1) % period == 0 and t_len > budget_k + recent_b


def run_decode(n_layers, leaders, K0, V0, t0, q_steps, k_new_steps,
               v_new_steps, evict=None, scale=None):
    """Reference trajectory of the whole decode loop on a small problem.

    K0, V0: [n_slots][nb][Hkv][T0][d] initial leader caches (t0 rows used).
    q_steps: [steps][n_layers][nb][Hq][d]; k_new_steps, v_new_steps:
    [steps][n_slots][nb][Hkv][d], the rows each leader appends per step.
    evict: None or a dict with K, B, N_v, period, w, seed (pass r uses
    seed + r).  Window queries for a leader are its own last w queries.
    Returns per-step outputs [steps][n_layers][nb][Hq][d], the final caches,
    the final length and a list of (step, slot, b, j, kept) records."""
    src_layer, src_slot = share_map(n_layers, leaders)
    n_slots = len(leaders)
    K0 = np.asarray(K0, dtype=np.float64)
    V0 = np.asarray(V0, dtype=np.float64)
    _, nb, hkv, _, d = K0.shape
    steps = len(q_steps)
    cap = t0 + steps
    Kc = np.zeros((n_slots, nb, hkv, cap, d))
    Vc = np.zeros((n_slots, nb, hkv, cap, d))
    Kc[:, :, :, :t0] = K0[:, :, :, :t0]
    Vc[:, :, :, :t0] = V0[:, :, :, :t0]
    t_len = t0
    outs = []
    records = []
    r = 0
    hq = np.asarray(q_steps).shape[3]
    g = hq // hkv
    for s in range(steps):
        for slot in range(n_slots):
            for b in range(nb):
                for j in range(hkv):
                    Kc[slot, b, j, t_len] = k_new_steps[s][slot][b][j]
                    Vc[slot, b, j, t_len] = v_new_steps[s][slot][b][j]
        t_len += 1
        q = np.asarray(q_steps[s], dtype=np.float64)
        o, _ = decode_attention(q, Kc, Vc, src_slot, hkv, t_len, scale)
        outs.append(o)
        if evict and eviction_due(s, evict["period"], t_len, evict["K"], evict["B"]):
            w = evict["w"]
            newK = np.zeros_like(Kc)
            newV = np.zeros_like(Vc)
            n_keep = None
            for slot, layer in enumerate(leaders):
                for b in range(nb):
                    for j in range(hkv):
                        qo = np.stack([np.asarray(q_steps[s - w + 1 + i], dtype=np.float64)
                                       [layer, b, j * g:(j + 1) * g] for i in range(w)])
                        sc = window_score(qo, Kc[slot, b, j], t_len, scale)
                        vr = value_range(Vc[slot, b, j, :t_len])
                        kept = select(sc, vr, t_len, evict["K"], evict["B"], evict["N_v"],
                                      evict["seed"] + r, layer, b, j)
                        records.append((s, slot, b, j, kept))
                        kk, vv = compact(Kc[slot, b, j], Vc[slot, b, j], kept)
                        n_keep = len(kept)
                        newK[slot, b, j, :n_keep] = kk
                        newV[slot, b, j, :n_keep] = vv
            Kc, Vc, t_len = newK, newV, n_keep
            r += 1
    return np.stack(outs), Kc, Vc, t_len, records

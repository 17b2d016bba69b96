"""Ragged batches for the oracle: per-sequence lengths and per-sequence
eviction steps (test infrastructure).

TEST INFRASTRUCTURE ONLY: tests/, the package's smoke check and the CPU
baseline leg of bench.py are the only code that may import it.  It shares no
code with the HIP library.

The pages state the method for one sequence.  VASE summary (gist.science
2606.03928), §2: a sequence's cache is pruned back to K + B rows every
`period` decode steps once it holds more than K + B rows; nothing on the
pages couples two sequences of a batch.  The reading fixed here for a batch
whose sequences differ in length and in where they stand in their period:

* every sequence b is the single-sequence method on its own rows: attention,
  window score, value range, selection and compaction see only rows
  [0, T_b) of that sequence;
* sequence b has a phase p_b: after decode step s (0-based, all sequences
  step together) it runs an eviction pass when (s + 1 + p_b) is a multiple
  of the period, it has decoded at least w steps (its observation window
  exists), and T_b > K + B.  All phases 0 give the uniform schedule;
* the sequences due after one step form one pass: pass r (counted over the
  steps that have a due sequence; the prompt compression is pass 0) draws
  with seed + r, and the Philox counter's batch word is the sequence's index
  b in the batch, whichever sequences share the pass;
* a window row that sees no cached row (a sequence shorter than the window)
  adds nothing to the score.
"""
import math

import numpy as np

from .kvc_oracle import attention, value_range, select, compact


def window_score_ragged(q_obs, K, t_len, scale=None):
    """Window score of one slab with t_len rows, for any t_len >= 0.

    Window row i (of w, oldest first) sees rows t <= t_len - w + i; a row
    that sees none contributes nothing.  For t_len >= w this is the window
    score of the single-sequence method (VASE §2.B)."""
    q_obs = np.asarray(q_obs, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)[:t_len]
    w, g, d = q_obs.shape
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    score = np.zeros(t_len)
    for i in range(w):
        visible = t_len - w + i + 1
        if visible <= 0:
            continue
        s = (q_obs[i] @ K[:visible].T) * scale
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        p /= p.sum(axis=1, keepdims=True)
        score[:visible] += p.sum(axis=0)
    return score


def eviction_due_seq(step, period, phase, w, t_len, budget_k, recent_b):
    """Whether a sequence of phase `phase` and length t_len runs an eviction
    pass after decode step `step`."""
    return ((step + 1 + phase) % period == 0 and step + 1 >= w
            and t_len > budget_k + recent_b)


def lengths_schedule(t0, n_steps, evict, initial_pass=True):
    """Host-side length bookkeeping of the ragged schedule, no data: returns
    (lengths after each step's append [n_steps][nb], the due sequences of each
    step (list of lists), lengths after each step [n_steps][nb]).  With an
    eviction config and the initial pass the prompt lengths are first cut to
    min(t0_b, K + B)."""
    nb = len(t0)
    cur = np.array(t0, dtype=np.int64)
    if evict and initial_pass:
        cur = np.minimum(cur, evict["K"] + evict["B"])
    att = np.zeros((n_steps, nb), dtype=np.int64)
    end = np.zeros((n_steps, nb), dtype=np.int64)
    due = []
    for s in range(n_steps):
        cur = cur + 1
        att[s] = cur
        d = []
        if evict:
            for b in range(nb):
                if eviction_due_seq(s, evict["period"], evict["phase"][b], evict["w"], cur[b],
                                    evict["K"], evict["B"]):
                    d.append(b)
            for b in d:
                cur[b] = min(cur[b], evict["K"] + evict["B"])
        due.append(d)
        end[s] = cur
    return att, due, end


def run_decode_ragged(n_layers, leaders, K0, V0, t0, q_steps, k_new_steps, v_new_steps,
                      evict=None, scale=None, initial_q_obs=None):
    """Reference trajectory of a ragged batch.

    K0, V0: [n_slots][nb][Hkv][>=max t0][d] prompt caches; t0[b]: prompt rows
    of sequence b.  q_steps: [steps][n_layers][nb][Hq][d]; k_new_steps,
    v_new_steps: [steps][n_slots][nb][Hkv][d].  evict: None or dict(K, B,
    N_v, period, w, seed, phase=[nb]).  With evict and initial_q_obs, the
    prompt of every sequence is first compressed by pass 0 (window scores
    from initial_q_obs[slot] = [w][nb][Hq][d], the last prompt queries of
    the leader; a sequence of at most K + B rows keeps all of them) and the
    periodic passes count from 1; without initial_q_obs they count from 0.
    Returns (outputs [steps][n_layers][nb][Hq][d], final caches as per-slot,
    per-sequence lists of (K, V) arrays, final lengths, records of
    (step, slot, b, j, kept)); step -1 marks pass 0."""
    from .kvc_oracle import share_map
    _, src_slot = share_map(n_layers, leaders)
    n_slots = len(leaders)
    K0 = np.asarray(K0, dtype=np.float64)
    V0 = np.asarray(V0, dtype=np.float64)
    _, nb, hkv, _, d = K0.shape
    hq = np.asarray(q_steps).shape[3]
    g = hq // hkv
    # per (slot, b, j) row lists
    Kc = [[[K0[s, b, j, :t0[b]].copy() for j in range(hkv)] for b in range(nb)]
          for s in range(n_slots)]
    Vc = [[[V0[s, b, j, :t0[b]].copy() for j in range(hkv)] for b in range(nb)]
          for s in range(n_slots)]
    lens = list(int(x) for x in t0)
    records = []
    r = 0
    if evict and initial_q_obs is not None:
        for slot, layer in enumerate(leaders):
            for b in range(nb):
                for j in range(hkv):
                    T = lens[b]
                    qo = np.asarray(initial_q_obs[slot], dtype=np.float64)[:, b, j * g:(j + 1) * g]
                    sc = window_score_ragged(qo, Kc[slot][b][j], T, scale)
                    vr = value_range(Vc[slot][b][j][:T])
                    kept = select(sc, vr, T, evict["K"], evict["B"], evict["N_v"],
                                  evict["seed"] + r, layer, b, j)
                    records.append((-1, slot, b, j, kept))
                    Kc[slot][b][j], Vc[slot][b][j] = compact(Kc[slot][b][j], Vc[slot][b][j], kept)
        lens = [min(T, evict["K"] + evict["B"]) for T in lens]
        r += 1
    outs = []
    steps = len(q_steps)
    for s in range(steps):
        for slot in range(n_slots):
            for b in range(nb):
                for j in range(hkv):
                    Kc[slot][b][j] = np.vstack([Kc[slot][b][j],
                                                np.asarray(k_new_steps[s][slot][b][j],
                                                           dtype=np.float64)[None]])
                    Vc[slot][b][j] = np.vstack([Vc[slot][b][j],
                                                np.asarray(v_new_steps[s][slot][b][j],
                                                           dtype=np.float64)[None]])
        lens = [T + 1 for T in lens]
        q = np.asarray(q_steps[s], dtype=np.float64)
        o = np.zeros((n_layers, nb, hq, d))
        for l in range(n_layers):
            for b in range(nb):
                for j in range(hkv):
                    heads = slice(j * g, (j + 1) * g)
                    o[l, b, heads], _ = attention(q[l, b, heads], Kc[src_slot[l]][b][j],
                                                  Vc[src_slot[l]][b][j], scale)
        outs.append(o)
        if not evict:
            continue
        due = [b for b in range(nb)
               if eviction_due_seq(s, evict["period"], evict["phase"][b], evict["w"], lens[b],
                                   evict["K"], evict["B"])]
        if not due:
            continue
        w = evict["w"]
        for slot, layer in enumerate(leaders):
            for b in due:
                for j in range(hkv):
                    T = lens[b]
                    qo = np.stack([np.asarray(q_steps[s - w + 1 + i], dtype=np.float64)
                                   [layer, b, j * g:(j + 1) * g] for i in range(w)])
                    sc = window_score_ragged(qo, Kc[slot][b][j], T, scale)
                    vr = value_range(Vc[slot][b][j])
                    kept = select(sc, vr, T, evict["K"], evict["B"], evict["N_v"],
                                  evict["seed"] + r, layer, b, j)
                    records.append((s, slot, b, j, kept))
                    Kc[slot][b][j], Vc[slot][b][j] = compact(Kc[slot][b][j], Vc[slot][b][j], kept)
        for b in due:
            lens[b] = min(lens[b], evict["K"] + evict["B"])
        r += 1
    return np.stack(outs) if outs else np.zeros((0,)), (Kc, Vc), lens, records

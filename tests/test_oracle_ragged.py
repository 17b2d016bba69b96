"""Pins of the ragged-batch oracle (oracle/ragged.py): the window score of
sequences shorter than the window, reduction of the ragged trajectory to the
uniform one, per-sequence independence and the length schedule.

VASE summary (gist.science 2606.03928), §2 states the method per sequence;
the ragged reading (phases, pass numbering, batch word of the counter) is
the one oracle/ragged.py documents."""
import math

import numpy as np
import pytest

import oracle
from oracle import ragged


def rng(s):
    return np.random.default_rng(s)


def brute_window_score(q_obs, K, t_len):
    """Python loops, math.exp: window row i sees rows t <= t_len - w + i."""
    w, g, d = q_obs.shape
    sc = 1.0 / math.sqrt(d)
    out = [0.0] * t_len
    for i in range(w):
        vis = t_len - w + i + 1
        if vis <= 0:
            continue
        for h in range(g):
            logits = [sum(q_obs[i][h][c] * K[t][c] for c in range(d)) * sc for t in range(vis)]
            m = max(logits)
            e = [math.exp(x - m) for x in logits]
            z = sum(e)
            for t in range(vis):
                out[t] += e[t] / z
    return np.array(out)


@pytest.mark.parametrize("T,w,g", [(0, 3, 2), (1, 4, 1), (3, 5, 2), (5, 5, 3), (9, 4, 2)])
def test_window_score_short_sequences_brute_force(T, w, g):
    G = rng(T * 10 + w)
    q = G.normal(size=(w, g, 6))
    K = G.normal(size=(max(T, 1), 6))
    got = ragged.window_score_ragged(q, K, T)
    np.testing.assert_allclose(got, brute_window_score(q, K, T), rtol=1e-12, atol=1e-14)
    # every window row that sees a row adds one unit per head
    assert got.sum() == pytest.approx(g * min(w, T), rel=1e-12, abs=1e-12)


def test_window_score_reduces_to_single_sequence_score():
    G = rng(1)
    q = G.normal(size=(8, 4, 32))
    K = G.normal(size=(100, 32))
    for T in (8, 9, 50, 100):
        assert np.array_equal(ragged.window_score_ragged(q, K, T), oracle.window_score(q, K, T))


def test_due_rule():
    # phase 0 is the uniform rule once the window exists
    for s in range(40):
        for T in (10, 30):
            uni = oracle.eviction_due(s, 8, T, 16, 4)
            assert ragged.eviction_due_seq(s, 8, 0, 5, T, 16, 4) == (uni and s + 1 >= 5)
    # a phase shifts the steps: (s + 1 + p) % period == 0
    steps = [s for s in range(40) if ragged.eviction_due_seq(s, 8, 3, 2, 100, 16, 4)]
    assert steps == [4, 12, 20, 28, 36]


def problem(seed, L=4, leaders=(0, 2), nb=3, hq=4, hkv=2, d=16, Tmax=40, steps=14):
    G = rng(seed)
    n_slots = len(leaders)
    K0 = G.normal(size=(n_slots, nb, hkv, Tmax, d))
    V0 = G.normal(size=(n_slots, nb, hkv, Tmax, d))
    V0[:, :, :, ::7] *= 20                      # some large-range rows
    q = G.normal(size=(steps, L, nb, hq, d))
    kn = G.normal(size=(steps, n_slots, nb, hkv, d))
    vn = G.normal(size=(steps, n_slots, nb, hkv, d))
    return L, list(leaders), K0, V0, q, kn, vn


def test_uniform_batch_reduces_to_uniform_trajectory():
    L, leaders, K0, V0, q, kn, vn = problem(2)
    nb = K0.shape[1]
    ev = dict(K=20, B=4, N_v=3, period=4, w=3, seed=9)
    o1, K1, V1, t1, rec1 = oracle.run_decode(L, leaders, K0, V0, 30, q, kn, vn, ev)
    o2, (K2, V2), t2, rec2 = ragged.run_decode_ragged(L, leaders, K0, V0, [30] * nb, q, kn, vn,
                                                      dict(ev, phase=[0] * nb))
    assert np.array_equal(o1, o2)
    assert t2 == [t1] * nb
    assert len(rec1) == len(rec2)
    for a, b in zip(rec1, rec2):
        assert a[:4] == b[:4] and np.array_equal(a[4], b[4])
    for s in range(len(leaders)):
        for b in range(nb):
            for j in range(K0.shape[2]):
                assert np.array_equal(K1[s, b, j, :t1], K2[s][b][j])
                assert np.array_equal(V1[s, b, j, :t1], V2[s][b][j])


def test_longest_sequence_matches_its_solo_run():
    """Same phases, sequence 0 longest: every pass that touches another
    sequence also touches sequence 0, so its pass numbers, keys and outputs
    are those of a batch of one."""
    L, leaders, K0, V0, q, kn, vn = problem(3)
    ev = dict(K=16, B=4, N_v=2, period=4, w=3, seed=4)
    t0 = [37, 12, 25]
    o, (Kc, Vc), lens, rec = ragged.run_decode_ragged(L, leaders, K0, V0, t0, q, kn, vn,
                                                      dict(ev, phase=[0, 0, 0]))
    o1, K1, V1, t1, rec1 = oracle.run_decode(L, leaders, K0[:, :1], V0[:, :1], 37, q[:, :, :1],
                                             kn[:, :, :1], vn[:, :, :1], ev)
    assert np.array_equal(o[:, :, 0], o1[:, :, 0])
    assert lens[0] == t1
    mine = [r for r in rec if r[2] == 0]
    assert len(mine) == len(rec1)
    for a, b in zip(mine, rec1):
        assert a[0] == b[0] and np.array_equal(a[4], b[4])


def test_sequences_do_not_interact():
    """Changing one sequence's data changes nothing of another's, as long as
    the pass numbering (the schedule) is unchanged."""
    L, leaders, K0, V0, q, kn, vn = problem(5)
    ev = dict(K=16, B=4, N_v=2, period=5, w=3, seed=1, phase=[0, 2, 4])
    t0 = [30, 22, 40]
    base = ragged.run_decode_ragged(L, leaders, K0, V0, t0, q, kn, vn, ev)
    K0b, V0b, qb, knb = K0.copy(), V0.copy(), q.copy(), kn.copy()
    G = rng(77)
    K0b[:, 1] = G.normal(size=K0b[:, 1].shape)
    V0b[:, 1] = G.normal(size=V0b[:, 1].shape)
    qb[:, :, 1] = G.normal(size=qb[:, :, 1].shape)
    knb[:, :, 1] = G.normal(size=knb[:, :, 1].shape)
    other = ragged.run_decode_ragged(L, leaders, K0b, V0b, t0, qb, knb, vn, ev)
    for b in (0, 2):
        assert np.array_equal(base[0][:, :, b], other[0][:, :, b])
        ra = [r for r in base[3] if r[2] == b]
        rb = [r for r in other[3] if r[2] == b]
        assert len(ra) == len(rb) and all(np.array_equal(x[4], y[4]) for x, y in zip(ra, rb))
    assert not np.array_equal(base[0][:, :, 1], other[0][:, :, 1])


def test_schedule_lengths_and_kept_counts():
    L, leaders, K0, V0, q, kn, vn = problem(6, steps=24, Tmax=60)
    nb = K0.shape[1]
    ev = dict(K=20, B=4, N_v=3, period=6, w=4, seed=2, phase=[0, 2, 5])
    t0 = [60, 10, 24]
    qi = [q[-4:, leaders[s]] for s in range(len(leaders))]     # stand-in prompt window
    o, (Kc, Vc), lens, rec = ragged.run_decode_ragged(L, leaders, K0, V0, t0, q, kn, vn, ev,
                                                      initial_q_obs=qi)
    att, due, end = ragged.lengths_schedule(t0, len(q), ev)
    assert lens == list(end[-1])
    # pass 0: every slab of every sequence, min(t0, K + B) rows kept
    p0 = [r for r in rec if r[0] == -1]
    assert len(p0) == len(leaders) * nb * K0.shape[2]
    for r in p0:
        assert len(r[4]) == min(t0[r[2]], 24)
    # periodic passes: exactly the due sequences, K + B rows kept each
    for s in range(len(q)):
        here = sorted({r[2] for r in rec if r[0] == s})
        assert here == due[s]
        for b in due[s]:
            assert att[s][b] > 24 and (s + 1 + ev["phase"][b]) % 6 == 0
        for r in rec:
            if r[0] == s:
                assert len(r[4]) == 24
    # the phases put the sequences' passes on different steps
    steps_of = [{s for s in range(len(q)) if b in due[s]} for b in range(nb)]
    assert steps_of[0] and steps_of[2] and not (steps_of[0] & steps_of[2])
    # after its first pass a sequence never holds more than K + B + period
    # rows (before it, the window condition may hold a pass back)
    for b in range(nb):
        first = min(steps_of[b]) if steps_of[b] else len(q)
        assert all(att[s][b] <= 24 + 6 for s in range(first + 1, len(q)))
    assert att[6][2] == 31 and 6 in steps_of[2]    # phase 5: step 0 had no window yet
    for s in range(len(leaders)):
        for b in range(nb):
            assert all(len(Kc[s][b][j]) == lens[b] for j in range(K0.shape[2]))

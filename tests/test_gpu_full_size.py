"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (the same Decoder schedule, shapes and calls), on sampled outputs the
oracle computes slab by slab.

Tolerances as in test_gpu_parity.py: bf16 attention max abs error <= 2e-2;
kept sets exact except rows within 1e-6 (relative) of the oracle's sampling
cutoff, which are counted and printed; compaction bit-exact."""
import sys

import numpy as np
import pytest
import torch

import oracle
import kvc_synth
import decode_attention_kvc_amd as kvc
from decode_attention_kvc_amd.loop import Decoder
from helpers import band_compare

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def make_state(L, leaders, nb, hq, hkv, t0, ev, steps, seed=0, t_cap=None, v_layout="tiles"):
    """The bench's setup: a prompt cache (v_layout "rows": a prefill's layout,
    as the bench holds its prompts), query/append pools, a Decoder."""
    n_slots = len(leaders)
    big = kvc.Cache.empty(n_slots, nb, hkv, t_cap or t0, device=DEV, v_layout=v_layout)
    for s in range(n_slots):
        K, V, _, _ = kvc_synth.kv_slot(nb, hkv, t0, device=DEV, seed=seed * 100 + s)
        big.fill(s, K, V)
        del K, V
    qpool = kvc_synth.queries((L, steps, nb, hq, 128), device=DEV, seed=seed + 1)
    lsepool = torch.zeros((L, steps, nb, hq), device=DEV)
    knew = kvc_synth.queries((steps, n_slots, nb, hkv, 128), device=DEV, seed=seed + 2)
    vnew = kvc_synth.queries((steps, n_slots, nb, hkv, 128), device=DEV, seed=seed + 3)
    return big, qpool, lsepool, knew, vnew


def slab64(cache, slot, b, j):
    K = cache.k[slot, b, j, : cache.t_len].double().cpu().numpy()
    V = cache.v_rows(slot)[b, j].double().cpu().numpy()
    return K, V


def check_attention_samples(dec, qpool, out, s, samples, L, hq, hkv):
    """Sampled (layer, b, kv head) rows of the last step's outputs."""
    g = hq // hkv
    worst = 0.0
    for (layer, b, j) in samples:
        slot = dec.src_slot[layer]
        K, V = slab64(dec.cache, slot, b, j)
        q = qpool[layer, s, b, j * g:(j + 1) * g].double().cpu().numpy()
        ref, _ = oracle.attention(q, K, V)
        got = out[layer, b, j * g:(j + 1) * g].double().cpu().numpy()
        worst = max(worst, float(np.abs(got - ref).max()))
    return worst


def test_llama31_8b_combined_full_size():
    """32 layers, 8 leaders, batch 16, 32K prompt -> K+B = 8320, per-layer."""
    L, leaders, nb, hq, hkv, t0 = 32, list(range(0, 32, 4)), 16, 32, 8, 32768
    ev = dict(K=8192, B=128, N_v=128, w=32, period=128, seed=0)
    steps = 4
    say("full-size combined: setup (prompt cache with value rows)")
    big, qpool, lsepool, knew, vnew = make_state(L, leaders, nb, hq, hkv, t0, ev, steps,
                                                 v_layout="rows")
    cap = ev["K"] + ev["B"] + ev["period"]
    cache = kvc.Cache.empty(len(leaders), nb, hkv, cap, device=DEV)
    spare = kvc.Cache.empty(len(leaders), nb, hkv, cap, device=DEV)
    dec = Decoder(L, leaders, big, cache, hq, evict=ev)
    q_init = [kvc_synth.queries((ev["w"], nb, hq, 128), device=DEV, seed=50 + i)
              for i in range(len(leaders))]
    # Keep the sampled prompt slabs on the host for the initial-pass check.
    picks = [(0, 0, 0), (3, 7, 5), (7, 15, 7)]
    pre = {(s, b, j): slab64(big, s, b, j) for (s, b, j) in picks}
    dec.initial_pass(q_init)
    dec.spare = spare
    torch.cuda.synchronize()
    assert dec.cache.t_len == 8320
    say("full-size combined: initial pass done; checking sampled slabs")
    g = hq // hkv
    ties = 0
    for (s, b, j) in picks:
        K0, V0 = pre[(s, b, j)]
        qo = q_init[s][:, b, j * g:(j + 1) * g].double().cpu().numpy()
        sc = oracle.window_score(qo, K0, t0)
        vr = oracle.value_range(V0)
        d = oracle.select_detail(sc, vr, t0, ev["K"], ev["B"], ev["N_v"], ev["seed"] + 0,
                                 leaders[s], b, j)
        K1, V1 = slab64(dec.cache, s, b, j)
        # the compacted slab is a gather of the prompt slab: recover its rows
        kept = _rows_of(K0, K1)
        t, bad = band_compare(kept, d)
        ties += t
        assert bad == 0, (s, b, j)
        assert np.array_equal(V1, V0[kept])
    say(f"  initial pass: kept sets match, {ties} ties within the band")
    out = torch.empty((L, nb, hq, 128), device=DEV)
    for s in range(steps):
        dec.step(s, qpool, lsepool, knew, vnew, out)
    torch.cuda.synchronize()
    assert dec.cache.t_len == 8320 + steps
    samples = [(0, 0, 0), (1, 3, 2), (5, 15, 7), (30, 8, 4), (31, 15, 0)]
    worst = check_attention_samples(dec, qpool, out, steps - 1, samples, L, hq, hkv)
    say(f"  decode step at T={dec.cache.t_len}: max |o - ref| = {worst:.2e}")
    assert worst <= 2e-2


def _rows_of(K0, K1):
    """Indices i with K1[r] == K0[i[r]] (rows are distinct random draws)."""
    keys0 = {K0[i].tobytes(): i for i in range(len(K0))}
    return np.array([keys0[K1[r].tobytes()] for r in range(len(K1))])


def test_qwen3_8b_rcla_full_size():
    """36 layers, 9 leaders, batch 1, 32K context; followers read leaders."""
    L, leaders, nb, hq, hkv, t0 = 36, list(range(0, 36, 4)), 1, 32, 8, 32768
    steps = 3
    say("full-size R-CLA: setup")
    big, qpool, lsepool, knew, vnew = make_state(L, leaders, nb, hq, hkv, t0, None, steps,
                                                 t_cap=t0 + 64)
    dec = Decoder(L, leaders, big, None, hq)
    out = torch.empty((L, nb, hq, 128), device=DEV)
    for s in range(steps):
        dec.step(s, qpool, lsepool, knew, vnew, out)
    torch.cuda.synchronize()
    assert dec.cache.t_len == t0 + steps
    # the appended rows landed in the leaders' slots
    assert torch.equal(dec.cache.k[2, :, :, t0 + 1], knew[1, 2])
    samples = [(0, 0, 0), (1, 0, 3), (3, 0, 7), (4, 0, 1), (22, 0, 5), (35, 0, 6)]
    worst = check_attention_samples(dec, qpool, out, steps - 1, samples, L, hq, hkv)
    say(f"  T={dec.cache.t_len}: max |o - ref| = {worst:.2e}")
    assert worst <= 2e-2


def test_qwen3_4b_vase_steady_eviction_full_size():
    """36 layers (all leaders), batch 8, steady state: 128 steps from K+B rows
    to the eviction at 4352 rows, scores from the decode log-normalisers."""
    L, leaders, nb, hq, hkv = 36, list(range(36)), 8, 32, 8
    ev = dict(K=4096, B=128, N_v=64, w=32, period=128, seed=7)
    t0, steps = ev["K"] + ev["B"], 128
    say("full-size VASE steady state: setup")
    big, qpool, lsepool, knew, vnew = make_state(L, leaders, nb, hq, hkv, t0, ev, steps,
                                                 t_cap=t0 + steps + 64)
    spare = kvc.Cache.empty(L, nb, hkv, t0 + steps + 64, device=DEV)
    dec = Decoder(L, leaders, big, spare, hq, evict=ev)
    out = torch.empty((L, nb, hq, 128), device=DEV)
    picks = [(0, 0, 0), (17, 3, 4), (35, 7, 7)]
    for s in range(steps):
        evicted = dec.step(s, qpool, lsepool, knew, vnew, out)
        assert evicted == (s == steps - 1)
    assert dec.cache.t_len == t0
    torch.cuda.synchronize()
    pre_t = t0 + steps                                # rows when the pass ran
    say("  eviction done; checking sampled slabs against the oracle")
    # The pre-eviction slab = prompt rows + the 128 appended rows.
    g = hq // hkv
    ties = 0
    for (layer, b, j) in picks:
        K0, V0, _, _ = kvc_synth.kv_slot(nb, hkv, t0, device=DEV, seed=0 * 100 + layer)
        Kp = torch.cat([K0[b, j], knew[:, layer, b, j]], 0).double().cpu().numpy()
        Vp = torch.cat([V0[b, j], vnew[:, layer, b, j]], 0).double().cpu().numpy()
        assert len(Kp) == pre_t
        qo = qpool[layer, steps - ev["w"]:steps, b, j * g:(j + 1) * g].double().cpu().numpy()
        sc = oracle.window_score(qo, Kp, pre_t)
        d = oracle.select_detail(sc, oracle.value_range(Vp), pre_t, ev["K"], ev["B"], ev["N_v"],
                                 ev["seed"] + 1, layer, b, j)
        K1, V1 = slab64(dec.cache, layer, b, j)
        kept = _rows_of(Kp, K1)
        t, bad = band_compare(kept, d)
        ties += t
        assert bad == 0, (layer, b, j)
        assert np.array_equal(V1, Vp[kept])
    say(f"  steady-state pass: kept sets match, {ties} ties within the band")


def test_qwen3_14b_long_initial_pass_full_size():
    """40 layers, 20 leaders, batch 4, 40/8 heads, 128K prompt -> 33024 rows."""
    L, leaders, nb, hq, hkv, t0 = 40, list(range(0, 40, 2)), 4, 40, 8, 131072
    ev = dict(K=32768, B=256, N_v=256, w=32, period=256, seed=3)
    steps = 2
    say("full-size long context: setup (43 GB prompt cache, value rows)")
    big, qpool, lsepool, knew, vnew = make_state(L, leaders, nb, hq, hkv, t0, ev, steps, seed=5,
                                                 v_layout="rows")
    cap = ev["K"] + ev["B"] + ev["period"]
    cache = kvc.Cache.empty(len(leaders), nb, hkv, cap, device=DEV)
    dec = Decoder(L, leaders, big, cache, hq, evict=ev)
    q_init = [kvc_synth.queries((ev["w"], nb, hq, 128), device=DEV, seed=70 + i)
              for i in range(len(leaders))]
    picks = [(0, 0, 0), (19, 3, 7)]
    pre = {(s, b, j): slab64(big, s, b, j) for (s, b, j) in picks}
    dec.initial_pass(q_init)
    torch.cuda.synchronize()
    assert dec.cache.t_len == 33024
    del big
    dec.spare = kvc.Cache.empty(len(leaders), nb, hkv, cap, device=DEV)
    g = hq // hkv
    ties = 0
    for (s, b, j) in picks:
        K0, V0 = pre[(s, b, j)]
        qo = q_init[s][:, b, j * g:(j + 1) * g].double().cpu().numpy()
        sc = oracle.window_score(qo, K0, t0)
        d = oracle.select_detail(sc, oracle.value_range(V0), t0, ev["K"], ev["B"], ev["N_v"],
                                 ev["seed"], leaders[s], b, j)
        K1, V1 = slab64(dec.cache, s, b, j)
        kept = _rows_of(K0, K1)
        t, bad = band_compare(kept, d)
        ties += t
        assert bad == 0, (s, b, j)
        assert np.array_equal(V1, V0[kept])
    say(f"  initial pass: kept sets match, {ties} ties within the band")
    out = torch.empty((L, nb, hq, 128), device=DEV)
    for s in range(steps):
        dec.step(s, qpool, lsepool, knew, vnew, out)
    torch.cuda.synchronize()
    worst = check_attention_samples(dec, qpool, out, steps - 1,
                                    [(0, 0, 0), (1, 2, 3), (38, 3, 7), (39, 1, 5)], L, hq, hkv)
    say(f"  decode at T={dec.cache.t_len}: max |o - ref| = {worst:.2e}")
    assert worst <= 2e-2


def _steady_pass(L, leaders, nb, hq, hkv, ev, picks, seed, label):
    """A steady-state periodic pass at full size, in the bench's launch
    configuration: the cache starts at K + B rows, the Decoder runs one
    period of steps with fused appends, and the pass after the last step
    scores the window with the decode log-normalisers (no compaction inside
    the window), selects and compacts every leader slab.  The sampled slabs
    are snapshotted one step before the pass; the oracle re-runs that pass
    (window score, range, selection with seed + 1, compaction) on the
    snapshot plus the appended row."""
    t0, P, w = ev["K"] + ev["B"], ev["period"], ev["w"]
    n_slots = len(leaders)
    say(f"steady pass {label}: setup ({t0} rows, {P} steps)")
    big, qpool, lsepool, knew, vnew = make_state(L, leaders, nb, hq, hkv, t0, ev, P, seed=seed,
                                                 t_cap=t0 + P + 64)
    spare = kvc.Cache.empty(n_slots, nb, hkv, t0 + P + 64, device=DEV)
    dec = Decoder(L, leaders, big, spare, hq, evict=ev)
    out = torch.empty((L, nb, hq, 128), device=DEV)
    for s in range(P - 1):
        assert not dec.step(s, qpool, lsepool, knew, vnew, out)
    torch.cuda.synchronize()
    snap = {p: slab64(dec.cache, *p) for p in picks}
    assert dec.step(P - 1, qpool, lsepool, knew, vnew, out)     # appends, then the pass
    torch.cuda.synchronize()
    pre_t = t0 + P
    assert dec.cache.t_len == t0
    say(f"  pass at {pre_t} rows done; checking {len(picks)} sampled slabs against the oracle")
    g = hq // hkv
    ties = 0
    for (slot, b, j) in picks:
        K0, V0 = snap[(slot, b, j)]
        Kp = np.concatenate([K0, knew[P - 1, slot, b, j].double().cpu().numpy()[None]], 0)
        Vp = np.concatenate([V0, vnew[P - 1, slot, b, j].double().cpu().numpy()[None]], 0)
        assert len(Kp) == pre_t
        leader = leaders[slot]
        qo = qpool[leader, P - w:P, b, j * g:(j + 1) * g].double().cpu().numpy()
        sc = oracle.window_score(qo, Kp, pre_t)
        d = oracle.select_detail(sc, oracle.value_range(Vp), pre_t, ev["K"], ev["B"], ev["N_v"],
                                 ev["seed"] + 1, leader, b, j)
        K1, V1 = slab64(dec.cache, slot, b, j)
        kept = _rows_of(Kp, K1)
        assert np.all(np.diff(kept) > 0)                 # ascending original rows
        t, bad = band_compare(kept, d)
        say(f"  slab (slot {slot}, b {b}, kv head {j}): {len(kept)} kept, {t} ties, "
            f"{bad} mismatches")
        ties += t
        assert bad == 0, (slot, b, j)
        assert np.array_equal(K1, Kp[kept]) and np.array_equal(V1, Vp[kept])
    say(f"  steady-state pass {label}: kept sets match, {ties} ties within the band")


def test_llama31_8b_combined_steady_pass_full_size():
    """32 layers, 8 leaders, batch 16, 32/8 heads: the pass at 8448 rows
    (K 8192, B 128, N_v 128, w 32, every 128 steps)."""
    ev = dict(K=8192, B=128, N_v=128, w=32, period=128, seed=0)
    _steady_pass(32, list(range(0, 32, 4)), 16, 32, 8, ev,
                 [(0, 0, 0), (3, 9, 4), (7, 15, 7)], seed=11, label="Llama-3.1-8B shape")


def test_qwen3_14b_long_steady_pass_full_size():
    """40 layers, 20 leaders, batch 4, 40/8 heads (g = 5, 160 window rows):
    the pass at 33280 rows (K 32768, B 256, N_v 256, w 32, every 256 steps)."""
    ev = dict(K=32768, B=256, N_v=256, w=32, period=256, seed=3)
    _steady_pass(40, list(range(0, 40, 2)), 4, 40, 8, ev,
                 [(0, 0, 0), (11, 2, 5), (19, 3, 7)], seed=13, label="Qwen3-14B shape")

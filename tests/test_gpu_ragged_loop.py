"""The ragged decode loop (loop.RaggedDecoder) against the oracle's ragged
trajectory (oracle/ragged.py).

float32 caches: the whole trajectory (every step's outputs, the final rows of
every sequence) is compared with run_decode_ragged, outputs within 1e-5
relative, rows bit-exact.  bf16 caches at larger sizes: every pass is
checked against the oracle applied to the GPU's own state just before it
(kept sets exact except rows within the score tolerance of the cutoff,
compaction bit-exact), and sampled outputs of every step within 1e-3."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import ragged
import kvc_synth
import decode_attention_kvc_amd as kvc
from decode_attention_kvc_amd.loop import RaggedDecoder, ragged_plan
from helpers import band_compare

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def setup(L, leaders, t0, hq, hkv, steps, ev, dtype, seed):
    nb, n_slots = len(t0), len(leaders)
    prompt = kvc.Cache.empty(n_slots, nb, hkv, max(t0), dtype=dtype, device=DEV)
    prompt.k.view(torch.int16).fill_(-1)
    prompt.v.view(torch.int16).fill_(-1)
    for s in range(n_slots):
        Kr, Vr, _, _ = kvc_synth.kv_slot(nb, hkv, max(t0), dtype=dtype, device=DEV,
                                         seed=seed * 10 + s)
        prompt.fill(s, Kr, Vr)
    qpool = kvc_synth.queries((L, steps, nb, hq, 128), dtype=dtype, device=DEV, seed=seed + 1)
    lsepool = torch.zeros((L, steps, nb, hq), device=DEV)
    knew = kvc_synth.queries((steps, n_slots, nb, hkv, 128), dtype=dtype, device=DEV, seed=seed + 2)
    vnew = kvc_synth.queries((steps, n_slots, nb, hkv, 128), dtype=dtype, device=DEV, seed=seed + 3)
    q_init = [kvc_synth.queries((ev["w"], nb, hq, 128), dtype=dtype, device=DEV, seed=seed + 10 + i)
              for i in range(n_slots)]
    plan = ragged_plan(t0, steps, ev)
    cache = kvc.Cache.empty(n_slots, plan["entries"], hkv, plan["peak"], dtype=dtype, device=DEV)
    cache.k.view(torch.int16).fill_(-1)
    cache.v.view(torch.int16).fill_(-1)
    return prompt, qpool, lsepool, knew, vnew, q_init, cache


def rows(cache, slot, entry, T):
    K = cache.k[slot, entry, :, :T].double().cpu().numpy()
    V = cache.v[slot, entry].transpose(-1, -2).reshape(cache.n_kv_heads, -1, 128)[:, :T]
    return K, V.double().cpu().numpy()


@pytest.mark.parametrize("mode", ["grouped", "per-layer"])
def test_ragged_trajectory_f32_matches_oracle(mode):
    L, leaders, hq, hkv = 4, [0, 2], 8, 2
    t0 = [300, 40, 150]
    ev = dict(K=64, B=16, N_v=8, period=8, w=4, seed=3, phase=[0, 3, 5])
    steps = 30
    say("ragged trajectory f32", mode)
    prompt, qpool, lsepool, knew, vnew, q_init, cache = setup(L, leaders, t0, hq, hkv, steps, ev,
                                                              torch.float32, seed=1)
    K0 = np.stack([prompt.k_rows(s).double().cpu().numpy() for s in range(len(leaders))])
    V0 = np.stack([prompt.v_rows(s).double().cpu().numpy() for s in range(len(leaders))])
    dec = RaggedDecoder(L, leaders, cache, hq, t0, steps, ev, mode=mode)
    dec.initial_pass(prompt, q_init)
    outs = []
    out = torch.empty((L, len(t0), hq, 128), device=DEV)
    n_pass = 0
    for s in range(steps):
        n_pass += dec.step(s, qpool, lsepool, knew, vnew, out)
        outs.append(out.clone())
    torch.cuda.synchronize()
    assert n_pass == len(dec.plan["passes"]) > 0
    qs = qpool.double().cpu().numpy().transpose(1, 0, 2, 3, 4)
    ref, (Kc, Vc), lens, rec = ragged.run_decode_ragged(
        L, leaders, K0, V0, t0, qs, knew.double().cpu().numpy(), vnew.double().cpu().numpy(),
        ev, initial_q_obs=[q.double().cpu().numpy() for q in q_init])
    got = torch.stack(outs).double().cpu().numpy()
    err = np.abs(got - ref).max()
    say(f"  max |o - ref| over {steps} steps: {err:.3e}")
    assert err <= 1e-5 * np.abs(ref).max()
    assert lens == dec.plan["final_len"]
    for s in range(len(leaders)):
        for b in range(len(t0)):
            Kg, Vg = rows(cache, s, dec.plan["final_entry"][b], lens[b])
            for j in range(hkv):
                assert np.array_equal(Kg[j], Kc[s][b][j])
                assert np.array_equal(Vg[j], Vc[s][b][j])


def _kept_from_rows(K0, K1):
    keys = {K0[i].tobytes(): i for i in range(len(K0))}
    return np.array([keys[K1[r].tobytes()] for r in range(len(K1))])


def test_ragged_loop_bf16_passes_stepwise():
    L, leaders, hq, hkv = 8, [0, 4], 32, 8
    t0 = [5000, 900, 3000, 2100]
    ev = dict(K=1024, B=64, N_v=32, period=32, w=32, seed=7, phase=[0, 8, 16, 24])
    steps = 70
    say("ragged loop bf16 stepwise")
    prompt, qpool, lsepool, knew, vnew, q_init, cache = setup(L, leaders, t0, hq, hkv, steps, ev,
                                                              torch.bfloat16, seed=4)
    dec = RaggedDecoder(L, leaders, cache, hq, t0, steps, ev)
    dec.initial_pass(prompt, q_init)
    torch.cuda.synchronize()
    plan = dec.plan
    kb = ev["K"] + ev["B"]
    g = hq // hkv
    out = torch.empty((L, len(t0), hq, 128), device=DEV)
    ties = worst = 0.0
    n_checked = 0
    for s in range(steps):
        p = plan["passes"].get(s)
        if p is not None:
            # the rows each due sequence holds after this step's append
            pre = {}
            for slot in range(len(leaders)):
                for b, e, Tb in zip(p["seqs"], p["src"], p["lens"]):
                    K, V = rows(cache, slot, e, Tb - 1)
                    K = np.concatenate([K, knew[s, slot, b].double().cpu().numpy()[:, None]], 1)
                    V = np.concatenate([V, vnew[s, slot, b].double().cpu().numpy()[:, None]], 1)
                    pre[(slot, b)] = (K, V)
        dec.step(s, qpool, lsepool, knew, vnew, out)
        torch.cuda.synchronize()
        # sampled outputs of this step against the state they attended to
        for (layer, b, j) in [(0, 0, 0), (3, 1, 5), (4, 2, 7), (7, 3, 2)]:
            slot = dec.src_slot[layer]
            Tb = plan["att_len"][s][b]
            if p is not None and b in p["seqs"]:
                K, V = pre[(slot, b)][0][j], pre[(slot, b)][1][j]
            else:
                K, V = rows(cache, slot, plan["att_idx"][s][b], Tb)
                K, V = K[j], V[j]
            ref, _ = oracle.attention(qpool[layer, s, b, j * g:(j + 1) * g].double().cpu().numpy(),
                                      K, V)
            worst = max(worst, np.abs(out[layer, b, j * g:(j + 1) * g].double().cpu().numpy()
                                      - ref).max())
        if p is None:
            continue
        for slot, leader in enumerate(leaders):
            for b, dst, Tb in zip(p["seqs"], p["dst"], p["lens"]):
                K, V = pre[(slot, b)]
                K1, V1 = rows(cache, slot, dst, kb)
                for j in range(hkv):
                    qo = np.stack([qpool[leader, s - ev["w"] + 1 + i, b, j * g:(j + 1) * g]
                                   .double().cpu().numpy() for i in range(ev["w"])])
                    sc = ragged.window_score_ragged(qo, K[j], Tb)
                    d = oracle.select_detail(sc, oracle.value_range(V[j]), Tb, ev["K"], ev["B"],
                                             ev["N_v"], ev["seed"] + p["round"], leader, b, j)
                    kept = _kept_from_rows(K[j], K1[j])
                    assert np.all(np.diff(kept) > 0)
                    assert np.array_equal(V1[j], V[j][kept])
                    t, bad = band_compare(kept, d, rel=2e-5)
                    ties += t
                    assert bad == 0, (s, slot, b, j)
                    n_checked += 1
    say(f"  {n_checked} slabs checked over {len(plan['passes'])} passes, {ties:.0f} ties; "
        f"max |o - ref| = {worst:.2e}")
    assert n_checked > 0 and worst <= 1e-3

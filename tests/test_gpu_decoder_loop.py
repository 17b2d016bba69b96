"""Whole decode trajectories of the uniform Decoder against the oracle's
run_decode, in float32: cross-layer sharing (followers read their leader's
slot), leader appends fused into the attention calls, and periodic eviction
passes whose window scores reuse the decode log-normalisers.  Every step's
outputs must match within 1e-5 of max |o| and the final caches (the
compacted rows, in ascending original order) bit for bit; a kept-set tie
would make the trajectories diverge, so this also checks that none occurs.
"""
import sys

import numpy as np
import pytest
import torch

import kvc_synth
import oracle
from helpers import make_cache, slab_np
from decode_attention_kvc_amd.loop import Decoder
import decode_attention_kvc_amd as kvc

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("mode", ["per-layer", "grouped", "per-layer-interleaved"])
def test_decoder_trajectory_f32_matches_oracle(mode):
    L, leaders, nb, hq, hkv = 6, [0, 2, 3], 2, 8, 2
    t0, steps = 90, 40
    ev = dict(K=48, B=8, N_v=4, w=6, period=16, seed=5)
    say("decoder trajectory f32", mode)
    n_slots = len(leaders)
    cache = make_cache(n_slots, nb, hkv, t0, t_cap=t0 + steps, dtype=torch.float32, seed=7)
    cache.t_len = t0
    spare = kvc.Cache.empty(n_slots, nb, hkv, t0 + steps, dtype=torch.float32, device=DEV)
    K0 = np.stack([slab_np(cache, s)[0] for s in range(n_slots)])
    V0 = np.stack([slab_np(cache, s)[1] for s in range(n_slots)])
    qpool = kvc_synth.queries((L, steps, nb, hq, 128), dtype=torch.float32, device=DEV, seed=1)
    lsepool = torch.zeros((L, steps, nb, hq), device=DEV)
    knew = kvc_synth.queries((steps, n_slots, nb, hkv, 128), dtype=torch.float32, device=DEV,
                             seed=2)
    vnew = kvc_synth.queries((steps, n_slots, nb, hkv, 128), dtype=torch.float32, device=DEV,
                             seed=3)
    # The oracle numbers the periodic passes from 0 (seed + r); the Decoder
    # reserves pass 0 for the initial compression of a prompt and starts the
    # periodic ones at 1, so it gets the seed one lower.
    dec = Decoder(L, leaders, cache, spare, hq, evict=dict(ev, seed=ev["seed"] - 1), mode=mode)
    out = torch.empty((L, nb, hq, 128), device=DEV)
    outs, n_pass = [], 0
    for s in range(steps):
        n_pass += dec.step(s, qpool, lsepool, knew, vnew, out)
        outs.append(out.clone())
    torch.cuda.synchronize()

    ref, Kc, Vc, t_len, rec = oracle.run_decode(
        L, leaders, K0, V0, t0, qpool.double().cpu().numpy().transpose(1, 0, 2, 3, 4),
        knew.double().cpu().numpy(), vnew.double().cpu().numpy(), evict=ev)
    assert n_pass == 2 == len({r[0] for r in rec})
    got = torch.stack(outs).double().cpu().numpy()
    err = np.abs(got - ref).max()
    say(f"  max |o - ref| over {steps} steps: {err:.3e}; final rows {dec.cache.t_len}")
    assert err <= 1e-5 * np.abs(ref).max()
    assert dec.cache.t_len == t_len == ev["K"] + ev["B"] + 8     # 8 appends after the last pass
    for s in range(n_slots):
        Kg, Vg = slab_np(dec.cache, s)
        assert np.array_equal(Kg, Kc[s][:, :, :t_len])
        assert np.array_equal(Vg, Vc[s][:, :, :t_len])

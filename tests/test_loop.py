"""Host schedule of the decode loop (decode_attention_kvc_amd.loop).

Stochastic KV Routing (aitrends.kr article on R-CLA), inference paragraph:
a follower reads its leader's KV, so within a step a follower's call must come
after the leader's append.  The call order is otherwise free; the interleaved
order exists so that consecutive calls read different slabs."""
import pytest
import torch

import decode_attention_kvc_amd as kvc
import kvc_synth
from decode_attention_kvc_amd.loop import Decoder


@pytest.mark.parametrize("L,leaders", [(8, [0, 3, 5]), (32, list(range(0, 32, 4))),
                                       (36, list(range(36))), (5, [0])])
def test_interleaved_order(L, leaders):
    c = kvc.Cache.empty(len(leaders), 1, 2, 64, device="cpu")
    d = Decoder(L, leaders, c, None, 8, mode="per-layer-interleaved")
    order = d.order["per-layer-interleaved"]
    assert sorted(order) == list(range(L))
    pos = {l: i for i, l in enumerate(order)}
    for l in range(L):
        assert pos[d.src_layer[l]] <= pos[l]          # leader (has appended) first
    if len(leaders) > 1:
        slots = [d.src_slot[l] for l in order]
        assert all(a != b for a, b in zip(slots, slots[1:]))
    assert d.order["per-layer"] == list(range(L))


def test_unknown_mode_rejected():
    c = kvc.Cache.empty(1, 1, 2, 64, device="cpu")
    with pytest.raises(ValueError):
        Decoder(2, [0], c, None, 8, mode="per-token")


@pytest.mark.gpu
def test_interleaved_matches_layer_order():
    """Same calls, other order: bit-identical outputs, lse and cache."""
    L, leaders, nb, hq, hkv, T0, steps = 12, [0, 4, 8], 2, 16, 4, 300, 3
    res = []
    for mode in ("per-layer", "per-layer-interleaved"):
        cache = kvc.Cache.empty(len(leaders), nb, hkv, T0 + 64, device="cuda")
        for s in range(len(leaders)):
            K, V, _, _ = kvc_synth.kv_slot(nb, hkv, T0, device="cuda", seed=s)
            cache.fill(s, K, V)
        qpool = kvc_synth.queries((L, steps, nb, hq, 128), device="cuda", seed=1)
        lsepool = torch.zeros((L, steps, nb, hq), device="cuda")
        knew = kvc_synth.queries((steps, len(leaders), nb, hkv, 128), device="cuda", seed=2)
        vnew = kvc_synth.queries((steps, len(leaders), nb, hkv, 128), device="cuda", seed=3)
        out = torch.empty((L, nb, hq, 128), device="cuda")
        dec = Decoder(L, leaders, cache, None, hq, mode=mode)
        for s in range(steps):
            dec.step(s, qpool, lsepool, knew, vnew, out)
        torch.cuda.synchronize()
        T = cache.t_len
        res.append((out.clone(), lsepool.clone(), cache.k[:, :, :, :T].clone(),
                     *[cache.v_rows(s) for s in range(len(leaders))]))
    for a, b in zip(*res):
        assert torch.equal(a, b)

"""Seeded random configurations of one whole eviction pass and the decode
attention after it, each step against the float64 oracle: window scores with
the fused value range (two passes, no decode log-normalisers), the selection
(fed the library's own scores, so that it is judged apart from their
rounding), the compaction, and attention over the compacted slot against
attention over the oracle's kept rows.  The shapes are drawn across the
boundaries of the kernels' tiling: head groups 1-8, windows 1-40, budgets
from one row to all of them, recent buffers and N_v from zero up, ragged
lengths, bfloat16 and float32."""
import sys

import numpy as np
import pytest
import torch

import oracle
import kvc_synth
import decode_attention_kvc_amd as kvc
from helpers import make_cache, slab_np, ws_tensor, to_np, band_compare

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CASES = 24


def draw(i):
    r = np.random.default_rng(9000 + i)
    dtype = torch.float32 if i % 6 == 5 else torch.bfloat16
    hkv = int(r.choice([1, 2, 4, 8]))
    g = int(r.integers(1, 9))
    nb = int(r.integers(1, 4))
    T = int(r.integers(40, 2500))
    w = int(r.integers(1, min(40, T) + 1))
    K = int(r.integers(1, T + 1)) if i % 8 != 7 else T      # every eighth case keeps all
    B = int(r.integers(0, 65))
    n_v = int(r.integers(0, K + 1)) if r.random() < 0.8 else 0
    seed = int(r.integers(0, 2**63))
    layer = int(r.integers(0, 64))
    return dtype, nb, hkv, g, T, w, K, B, n_v, seed, layer


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_eviction_pass_then_attention(i):
    dtype, nb, hkv, g, T, w, K, B, n_v, seed, layer = draw(i)
    hq = g * hkv
    print("fuzz", i, str(dtype)[6:], dict(nb=nb, hkv=hkv, g=g, T=T, w=w, K=K, B=B, n_v=n_v),
          file=sys.stderr, flush=True)
    src = make_cache(2, nb, hkv, T, dtype=dtype, seed=100 + i)
    q_obs = kvc_synth.queries((w, nb, hq, 128), dtype=dtype, device=DEV, seed=200 + i)
    # score and fused range
    score = torch.full((nb, hkv, T), float("nan"), device=DEV)
    rng = torch.full((nb, hkv, T), float("nan"), device=DEV)
    kvc.kvc_score(src, 1, q_obs, score, rng, None, ws_tensor(kvc.kvc_score_ws_bytes(src, hq, w)))
    torch.cuda.synchronize()
    Ks, Vs = slab_np(src, 1)
    qn = to_np(q_obs)
    for b in range(nb):
        for j in range(hkv):
            ref = oracle.window_score(qn[:, b, j * g:(j + 1) * g], Ks[b, j], T)
            got = score[b, j].double().cpu().numpy()
            nz = ref > 1e-30
            assert np.max(np.abs(got - ref)[nz] / ref[nz]) <= 1e-5, (b, j)
            assert np.array_equal(rng[b, j].cpu().numpy(),
                                  oracle.value_range(Vs[b, j]).astype(np.float32)), (b, j)
    # selection on the library's scores
    n_keep = min(T, K + B)
    kept = torch.full((nb, hkv, n_keep), -7, dtype=torch.int32, device=DEV)
    kvc.kvc_select(score, rng, nb, hkv, T, K, B, n_v, seed, layer, kept,
                   ws_tensor(kvc.kvc_select_ws_bytes(nb, hkv, T)))
    torch.cuda.synchronize()
    sc, rg, kp = to_np(score), rng.cpu().numpy(), kept.cpu().numpy()
    ties = 0
    for b in range(nb):
        for j in range(hkv):
            d = oracle.select_detail(sc[b, j], rg[b, j], T, K, B, n_v, seed, layer, b, j)
            assert len(kp[b, j]) == len(d["kept"])
            assert np.all(np.diff(kp[b, j]) > 0)
            t, bad = band_compare(kp[b, j], d)
            ties += t
            assert bad == 0, (b, j)
    # compaction into the other buffer, bit-exact
    dst = kvc.Cache.empty(2, nb, hkv, n_keep + 64, dtype=dtype, device=DEV)
    kvc.kvc_compact(src, 1, kept, n_keep, dst)
    torch.cuda.synchronize()
    dst.t_len = n_keep
    Kd, Vd = slab_np(dst, 1)
    for b in range(nb):
        for j in range(hkv):
            assert np.array_equal(Kd[b, j], Ks[b, j][kp[b, j]])
            assert np.array_equal(Vd[b, j], Vs[b, j][kp[b, j]])
    # attention over the compacted slot = attention over the kept rows
    q = kvc_synth.queries((1, nb, hq, 128), dtype=dtype, device=DEV, seed=300 + i)
    out = torch.full((1, nb, hq, 128), float("nan"), device=DEV)
    lse = torch.full((1, nb, hq), float("nan"), device=DEV)
    kvc.kvc_decode_attn(dst, q, [1], out, lse, ws_tensor(kvc.kvc_decode_attn_ws_bytes(dst, 1, hq)))
    torch.cuda.synchronize()
    on, ln, qq = to_np(out[0]), to_np(lse[0]), to_np(q[0])
    for b in range(nb):
        for j in range(hkv):
            ro, rl = oracle.attention(qq[b, j * g:(j + 1) * g], Ks[b, j][kp[b, j]],
                                      Vs[b, j][kp[b, j]])
            err = np.abs(on[b, j * g:(j + 1) * g] - ro).max()
            if dtype == torch.float32:
                assert err <= 1e-5 * np.abs(ro).max(), (b, j, err)
            else:
                assert err <= 2e-2, (b, j, err)
            assert np.abs(ln[b, j * g:(j + 1) * g] - rl).max() <= 1e-3, (b, j)
    print(f"  ties within the band: {ties}", file=sys.stderr, flush=True)

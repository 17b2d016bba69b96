"""GPU parity of ragged batches (per-sequence lengths, batch maps) for every
cache entry point, against the oracle on each sequence's own rows.

Tolerances are those of the uniform tests: bf16 attention max|o - o_ref| <=
1e-3 (bar 2e-2), lse 1e-4; float32 1e-5 relative; value ranges, appends and
compaction bit-exact; window scores 1e-5 relative; DKV scores as in the
uniform DKV test (a bound from each slab's sketch condition number); kept
sets exact except rows within 1e-6 of the cutoff.
Rows of an entry past its sequence's length hold NaN bit patterns, so a read
past the end shows up in the outputs."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import dkv as odkv
from oracle import ragged
import kvc_synth
import decode_attention_kvc_amd as kvc
from helpers import make_cache, slab_np, ws_tensor, to_np, band_compare, dkv_tolerance

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def bits(t):
    return t.contiguous().view(torch.int16)


def poison_tail(cache, entry, T):
    """NaN bits in rows [T, t_cap) of every slab of one batch entry."""
    cache.k[:, entry, :, T:].view(torch.int16).fill_(-1)
    tile, r = divmod(T, 32)
    if r:
        cache.v[:, entry, :, tile, :, r:].view(torch.int16).fill_(-1)
        tile += 1
    cache.v[:, entry, :, tile:].view(torch.int16).fill_(-1)


def ragged_setup(n_slots, nb_cap, hkv, T, idx, lens, dtype=torch.bfloat16, seed=0):
    cache = make_cache(n_slots, nb_cap, hkv, T, dtype=dtype, seed=seed)
    for e, L in zip(idx, lens):
        if 0 <= e < nb_cap:
            poison_tail(cache, e, L)
    K, V = zip(*[slab_np(cache, s) for s in range(n_slots)])   # [slot] -> [entry][j][T][d]
    bidx = torch.tensor(idx, dtype=torch.int32, device=DEV)
    slen = torch.tensor(lens, dtype=torch.int32, device=DEV)
    view = cache.seqs(bidx, slen, t_len=max(max(lens), 1))
    return cache, view, K, V


ATTN_CASES = [
    # (dtype, hq, hkv, nb_cap, batch_idx, lens, q_slot)
    (torch.bfloat16, 32, 8, 6, [4, 0, 5, 2, 1], [0, 1, 33, 1500, 777], [1, 0]),
    (torch.bfloat16, 32, 8, 3, [2, 0], [4097, 64], [0, 0, 0, 0]),        # grouped rows
    (torch.bfloat16, 40, 8, 4, [3, 1, 0, 2], [31, 8448, 2, 700], [1]),   # many splits
    (torch.bfloat16, 16, 4, 5, [1, 7, -1, 3], [300, 50, 60, 0], [0]),    # bad entries: empty
    (torch.float32, 8, 2, 3, [2, 0, 1], [1024, 65, 0], [0]),
    # 17 x 8 slabs: two workgroups per slab split the value channels
    (torch.bfloat16, 32, 8, 17, [16, 3, 0, 5, 9, 1, 2, 4, 6, 7, 8, 10, 11, 12, 13, -1, 15],
     [400, 0, 1, 33, 256, 257, 31, 32, 100, 7, 399, 64, 65, 200, 150, 90, 12], [1]),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: f"{str(c[0])[6:]}-{c[4]}-{c[5]}")
def test_ragged_decode_attn(case):
    dtype, hq, hkv, nb_cap, idx, lens, q_slot = case
    say("ragged attention", case)
    T = max(lens)
    cache, view, K, V = ragged_setup(2, nb_cap, hkv, T, idx, lens, dtype, seed=len(idx))
    nb, nq = len(idx), len(q_slot)
    q = kvc_synth.queries((nq, nb, hq, 128), dtype=dtype, device=DEV, seed=T)
    out = torch.full((nq, nb, hq, 128), float("nan"), device=DEV)
    lse = torch.full((nq, nb, hq), float("nan"), device=DEV)
    ws = ws_tensor(kvc.kvc_decode_attn_ws_bytes(view, nq, hq))
    kvc.kvc_decode_attn(view, q, q_slot, out, lse, ws)
    torch.cuda.synchronize()
    qn, o, l = to_np(q), to_np(out), to_np(lse)
    g = hq // hkv
    err = lerr = big = 0.0
    for i, s in enumerate(q_slot):
        for b, (e, Tb) in enumerate(zip(idx, lens)):
            empty = not (0 <= e < nb_cap) or Tb == 0
            for j in range(hkv):
                hs = slice(j * g, (j + 1) * g)
                if empty:
                    assert np.all(o[i, b, hs] == 0) and np.all(l[i, b, hs] == -np.inf)
                    continue
                ro, rl = oracle.attention(qn[i, b, hs], K[s][e, j, :Tb], V[s][e, j, :Tb])
                big = max(big, np.abs(ro).max())
                err = max(err, np.abs(o[i, b, hs] - ro).max())
                lerr = max(lerr, np.abs(l[i, b, hs] - rl).max())
    say(f"  max|o-ref| = {err:.3e}  max|lse-ref| = {lerr:.3e}")
    if dtype == torch.bfloat16:
        assert err <= 1e-3 and lerr <= 1e-4
    else:
        assert err <= 1e-5 * big and lerr <= 1e-5 * 10


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ragged_append_fused_and_standalone(dtype):
    say("ragged append", dtype)
    hkv, hq = (8, 32) if dtype == torch.bfloat16 else (2, 8)
    idx, lens = [2, 0, 3], [96, 1, 130]          # new row closes a tile / first row / mid tile
    cache, view, K, V = ragged_setup(2, 4, hkv, 160, idx, lens, dtype, seed=2)
    before = cache.k.clone(), cache.v.clone()
    nb = len(idx)
    kn = kvc_synth.queries((nb, hkv, 128), dtype=dtype, device=DEV, seed=5)
    vn = kvc_synth.queries((nb, hkv, 128), dtype=dtype, device=DEV, seed=6) * 3
    q = kvc_synth.queries((1, nb, hq, 128), dtype=dtype, device=DEV, seed=7)
    out = torch.empty((1, nb, hq, 128), device=DEV)
    ws = ws_tensor(kvc.kvc_decode_attn_ws_bytes(view, 1, hq))
    kvc.kvc_decode_attn(view, q, [1], out, None, ws, k_new=kn, v_new=vn, append_slot=1)
    torch.cuda.synchronize()
    expect_k, expect_v = before[0].clone(), before[1].clone()
    for b, (e, Tb) in enumerate(zip(idx, lens)):
        expect_k[1, e, :, Tb - 1] = kn[b]
        expect_v[1, e, :, (Tb - 1) // 32, :, (Tb - 1) % 32] = vn[b]
    assert torch.equal(bits(cache.k), bits(expect_k))
    assert torch.equal(bits(cache.v), bits(expect_v))
    qn, g = to_np(q), hq // hkv
    for b, (e, Tb) in enumerate(zip(idx, lens)):
        Kb = np.concatenate([K[1][e, :, :Tb - 1], to_np(kn)[b][:, None]], axis=1)
        Vb = np.concatenate([V[1][e, :, :Tb - 1], to_np(vn)[b][:, None]], axis=1)
        for j in range(hkv):
            ro, _ = oracle.attention(qn[0, b, j * g:(j + 1) * g], Kb[j], Vb[j])
            tol = 1e-3 if dtype == torch.bfloat16 else 1e-5 * np.abs(ro).max()
            assert np.abs(to_np(out[0, b, j * g:(j + 1) * g]) - ro).max() <= tol
    # standalone append into slot 0 of the same entries
    kvc.kvc_append(view, 0, vn, kn)
    torch.cuda.synchronize()
    for b, (e, Tb) in enumerate(zip(idx, lens)):
        assert torch.equal(bits(cache.k[0, e, :, Tb - 1]), bits(vn[b]))
        assert torch.equal(bits(cache.v[0, e, :, (Tb - 1) // 32, :, (Tb - 1) % 32]), bits(kn[b]))
    assert torch.equal(bits(cache.k[:, 1]), bits(before[0][:, 1]))     # an unused entry


SCORE_CASES = [
    # (dtype, hq, hkv, nb_cap, idx, lens, w, use_lse)
    (torch.bfloat16, 32, 8, 5, [3, 0, 4, 1], [1000, 20, 2113, 0], 32, False),
    (torch.bfloat16, 32, 8, 3, [1, 2], [33, 4352], 32, True),
    (torch.bfloat16, 16, 8, 2, [0, 1], [300, 7], 5, False),
    (torch.float32, 8, 2, 3, [2, 0], [1024, 100], 32, False),
]


def gpu_window_lse_ragged(view, slot, q_obs, lens):
    """Log-normalisers of the window rows as decode attention returns them
    (row i against the first T_b - w + i + 1 rows of sequence b)."""
    w, nb, hq, _ = q_obs.shape
    lse = torch.empty((w, nb, hq), device=DEV)
    out = torch.empty((1, nb, hq, 128), device=DEV)
    ws = ws_tensor(kvc.kvc_decode_attn_ws_bytes(view, 1, hq))
    for i in range(w):
        li = torch.tensor([max(0, L - w + i + 1) for L in lens], dtype=torch.int32, device=DEV)
        v = view.seqs(view.batch_idx, li, t_len=view.t_len)
        kvc.kvc_decode_attn(v, q_obs[i:i + 1], [slot], out, lse[i:i + 1], ws)
    torch.cuda.synchronize()
    return lse


@pytest.mark.parametrize("case", SCORE_CASES, ids=lambda c: f"{str(c[0])[6:]}-{c[5]}-w{c[6]}{'L' if c[7] else ''}")
def test_ragged_score_and_range(case):
    dtype, hq, hkv, nb_cap, idx, lens, w, use_lse = case
    say("ragged score", case)
    T = max(lens)
    cache, view, K, V = ragged_setup(2, nb_cap, hkv, T, idx, lens, dtype, seed=w)
    nb = len(idx)
    q_obs = kvc_synth.queries((w, nb, hq, 128), dtype=dtype, device=DEV, seed=T)
    lse = gpu_window_lse_ragged(view, 1, q_obs, lens) if use_lse else None
    score = torch.full((nb, hkv, T), float("nan"), device=DEV)
    rng = torch.full((nb, hkv, T), float("nan"), device=DEV)
    rng2 = torch.full((nb, hkv, T), float("nan"), device=DEV)
    ws = None if use_lse else ws_tensor(kvc.kvc_score_ws_bytes(view, hq, w))
    kvc.kvc_score(view, 1, q_obs, score, rng, lse, ws)
    kvc.kvc_value_range(view, 1, rng2)
    torch.cuda.synchronize()
    qn, g = to_np(q_obs), hq // hkv
    worst = 0.0
    for b, (e, Tb) in enumerate(zip(idx, lens)):
        for j in range(hkv):
            got = score[b, j].double().cpu().numpy()
            assert np.all(np.isnan(got[Tb:]))                        # not written
            assert np.all(np.isnan(rng[b, j, Tb:].cpu().numpy()))
            assert np.all(np.isnan(rng2[b, j, Tb:].cpu().numpy()))
            if Tb == 0:
                continue
            ref = ragged.window_score_ragged(qn[:, b, j * g:(j + 1) * g], K[1][e, j], Tb)
            rel = np.abs(got[:Tb] - ref) / np.maximum(ref, 1e-30)
            worst = max(worst, float(np.max(rel[ref > 1e-30])))
            assert got[:Tb].sum() == pytest.approx(g * min(w, Tb), rel=1e-4)
            rref = oracle.value_range(V[1][e, j, :Tb]).astype(np.float32)
            assert np.array_equal(rng[b, j, :Tb].cpu().numpy(), rref)
            assert np.array_equal(rng2[b, j, :Tb].cpu().numpy(), rref)
    say(f"  max relative score error {worst:.3e}")
    assert worst <= 1e-5


def test_ragged_select_seq_ids():
    say("ragged select")
    nb, hkv, T, K, B, Nv = 4, 2, 3000, 1024, 64, 32
    lens = [3000, 1000, 1088, 0]             # evicts / keeps all / exactly K + B / empty
    seq_id = [7, 2, 0, 5]
    g = torch.Generator(device=DEV).manual_seed(3)
    score = (torch.rand((nb, hkv, T), generator=g, device=DEV) ** 3) * 2.0
    rng = torch.rand((nb, hkv, T), generator=g, device=DEV) * 10
    n_keep = min(T, K + B)
    kept = torch.full((nb, hkv, n_keep), -7, dtype=torch.int32, device=DEV)
    kvc.kvc_select_seq(score, rng, nb, hkv, T, torch.tensor(lens, dtype=torch.int32, device=DEV),
                       torch.tensor(seq_id, dtype=torch.int32, device=DEV), K, B, Nv, 99, 3, kept,
                       ws_tensor(kvc.kvc_select_ws_bytes(nb, hkv, T)))
    torch.cuda.synchronize()
    sc, rg, kp = to_np(score), rng.cpu().numpy(), kept.cpu().numpy()
    for b, Tb in enumerate(lens):
        for j in range(hkv):
            m = min(Tb, K + B)
            assert np.all(kp[b, j, m:] == -1)
            if Tb == 0:
                continue
            d = oracle.select_detail(sc[b, j, :Tb], rg[b, j, :Tb], Tb, K, B, Nv, 99, 3,
                                     seq_id[b], j)
            ties, bad = band_compare(kp[b, j, :m], d)
            assert bad == 0 and len(kp[b, j, :m]) == len(d["kept"])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ragged_compact_between_entries(dtype):
    """Sequences move to other entries of the same cache (the ping-pong of
    per-sequence eviction); bit-exact gather, other entries untouched."""
    say("ragged compact", dtype)
    hkv, n_keep = 4, 300
    idx_src, idx_dst, lens = [0, 2, 4], [1, 3, 5], [1000, 120, 700]
    cache, view, K, V = ragged_setup(2, 6, hkv, 1000, idx_src, lens, dtype, seed=4)
    before_k, before_v = cache.k.clone(), cache.v.clone()
    nb = len(idx_src)
    gcpu = torch.Generator(device="cpu").manual_seed(1)
    kept = torch.full((nb, hkv, n_keep), -1, dtype=torch.int32)
    for b, Tb in enumerate(lens):
        m = min(Tb, n_keep)
        for j in range(hkv):
            kept[b, j, :m] = torch.randperm(Tb, generator=gcpu)[:m].sort().values.int()
    kept = kept.to(DEV)
    dst = cache.seqs(torch.tensor(idx_dst, dtype=torch.int32, device=DEV), None, t_len=n_keep)
    kvc.kvc_compact(view, 1, kept, n_keep, dst)
    torch.cuda.synchronize()
    Kc, Vc = slab_np(cache, 1)
    kc = kept.cpu().numpy()
    for b, Tb in enumerate(lens):
        m = min(Tb, n_keep)
        e, f = idx_src[b], idx_dst[b]
        for j in range(hkv):
            assert np.array_equal(Kc[f, j, :m], K[1][e, j, kc[b, j, :m]])
            assert np.array_equal(Vc[f, j, :m], V[1][e, j, kc[b, j, :m]])
        # rows past the kept count and the source entries are untouched
        assert torch.equal(bits(cache.k[1, f, :, m:]), bits(before_k[1, f, :, m:]))
        assert torch.equal(bits(cache.k[1, e]), bits(before_k[1, e]))
    assert torch.equal(bits(cache.k[0]), bits(before_k[0]))
    assert torch.equal(bits(cache.v[0]), bits(before_v[0]))


def test_ragged_dkv_scores():
    say("ragged dkv")
    hkv, rank = 4, 32
    idx, lens = [2, 0, 1], [4097, 20, 1000]
    cache, view, K, V = ragged_setup(1, 3, hkv, 4097, idx, lens, seed=8)
    nb, T = len(idx), max(lens)
    g = kvc_synth.queries((rank, 256), dtype=torch.bfloat16, device=DEV, seed=1)
    score = torch.full((nb, hkv, T), float("nan"), device=DEV)
    rng = torch.full((nb, hkv, T), float("nan"), device=DEV)
    kvc.kvc_dkv_score(view, 0, g, score, rng, ws_tensor(kvc.kvc_dkv_ws_bytes(view, rank)))
    torch.cuda.synchronize()
    G = g.double().cpu().numpy().T
    for b, (e, Tb) in enumerate(zip(idx, lens)):
        for j in range(hkv):
            got = score[b, j].double().cpu().numpy()
            assert np.all(np.isnan(got[Tb:]))
            ref = odkv.dkv_score(K[0][e, j, :Tb], V[0][e, j, :Tb], G)
            err = np.abs(got[:Tb] - ref)
            assert np.all(err <= dkv_tolerance(ref))
            assert got[:Tb].sum() == pytest.approx(min(Tb, rank), rel=1e-4)
            assert np.array_equal(rng[b, j, :Tb].cpu().numpy(),
                                  oracle.value_range(V[0][e, j, :Tb]).astype(np.float32))


def test_uniform_view_equals_plain_cache():
    """A map that is the identity, with every length t_len, gives the same
    bits as the plain cache."""
    say("identity view")
    nb, hq, hkv, T = 3, 32, 8, 1500
    cache = make_cache(1, nb, hkv, T, seed=12)
    view = cache.seqs(torch.arange(nb, dtype=torch.int32, device=DEV),
                      torch.full((nb,), T, dtype=torch.int32, device=DEV))
    q = kvc_synth.queries((2, nb, hq, 128), device=DEV, seed=3)
    outs = []
    for c in (cache, view):
        out = torch.empty((2, nb, hq, 128), device=DEV)
        lse = torch.empty((2, nb, hq), device=DEV)
        kvc.kvc_decode_attn(c, q, [0, 0], out, lse, ws_tensor(kvc.kvc_decode_attn_ws_bytes(c, 2, hq)))
        sc = torch.empty((nb, hkv, T), device=DEV)
        rg = torch.empty((nb, hkv, T), device=DEV)
        kvc.kvc_score(c, 0, q[:, :, :, :].repeat(16, 1, 1, 1), sc, rg, None,
                      ws_tensor(kvc.kvc_score_ws_bytes(c, hq, 32)))
        outs.append((out, lse, sc, rg))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("use_lse", [False, True])
def test_score_seq_reads_queries_through_the_index(use_lse):
    """kvc_score_seq over a subset of a batch's sequences, reading their
    window queries (and log-normalisers) through q_idx from the whole batch's
    arrays, equals kvc_score on the same queries gathered beforehand, bit for
    bit."""
    say("score_seq", use_lse)
    hkv, hq, w, T = 4, 16, 8, 900
    cache, view, K, V = ragged_setup(2, 6, hkv, T, [4, 1, 3], [900, 300, 650], seed=31)
    nb_all = 5
    q_all = kvc_synth.queries((w, nb_all, hq, 128), device=DEV, seed=32)
    lse_all = (torch.rand((w, nb_all, hq), device=DEV) * 3 + 5) if use_lse else None
    q_idx = torch.tensor([2, 0, 4], dtype=torch.int32, device=DEV)
    outs = []
    for mode in ("seq", "gathered"):
        sc = torch.full((3, hkv, T), float("nan"), device=DEV)
        rg = torch.full((3, hkv, T), float("nan"), device=DEV)
        ws = None if use_lse else ws_tensor(kvc.kvc_score_ws_bytes(view, hq, w))
        if mode == "seq":
            kvc.kvc_score_seq(view, 1, q_all, q_idx, sc, rg, lse_all, ws)
        else:
            li = q_idx.long()
            kvc.kvc_score(view, 1, q_all[:, li].contiguous(), sc, rg,
                          lse_all[:, li].contiguous() if use_lse else None, ws)
        outs.append((sc, rg))
    torch.cuda.synchronize()
    for b, L in enumerate([900, 300, 650]):
        assert torch.equal(outs[0][0][b, :, :L], outs[1][0][b, :, :L])
        assert torch.equal(outs[0][1][b, :, :L], outs[1][1][b, :, :L])

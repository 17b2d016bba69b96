"""Caches whose values are [t][d] rows (a prefill's layout, v_layout "rows"):
the prompt compression's calls read them -- value range, window score with the
fused range, compaction into the tiled decode layout (and, with no kept list,
a bulk ingest) -- with results equal bit for bit to the same calls on the
tiled form of the same rows, and to the oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
import kvc_synth
import decode_attention_kvc_amd as kvc
from decode_attention_kvc_amd.loop import Decoder
from helpers import make_cache, slab_np, ws_tensor, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def rows_twin(tiles):
    """A rows-layout cache holding the same logical rows as `tiles` (NaN bit
    patterns past t_len, as make_cache leaves them)."""
    r = kvc.Cache.empty(tiles.n_slots, tiles.nb_cap, tiles.n_kv_heads, tiles.t_cap,
                        dtype=tiles.dtype, device=DEV, v_layout="rows")
    r.k.view(torch.int16).fill_(-1)
    r.v.view(torch.int16).fill_(-1)
    for s in range(tiles.n_slots):
        r.fill(s, tiles.k_rows(s), tiles.v_rows(s))
    r.t_len = tiles.t_len
    return r


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T", [1, 63, 64, 1000, 4161])
def test_value_range_rows(dtype, T):
    say("range rows", dtype, T)
    tiles = make_cache(2, 2, 4, T, dtype=dtype, seed=T)
    rows = rows_twin(tiles)
    a = torch.full((2, 4, T), float("nan"), device=DEV)
    b = torch.full((2, 4, T), float("nan"), device=DEV)
    kvc.kvc_value_range(tiles, 1, a)
    kvc.kvc_value_range(rows, 1, b)
    torch.cuda.synchronize()
    _, V = slab_np(tiles, 1)
    ref = oracle.value_range(V.reshape(-1, 128)).astype(np.float32).reshape(2, 4, T)
    assert np.array_equal(b.cpu().numpy(), ref)
    assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,hq,w,T,use_lse", [
    (torch.bfloat16, 32, 32, 2113, False),
    (torch.bfloat16, 40, 32, 5000, False),
    (torch.float32, 8, 32, 1024, False),
])
def test_score_with_range_rows(dtype, hq, w, T, use_lse):
    say("score rows", dtype, hq, w, T)
    nb, hkv = 2, 8 if hq % 8 == 0 else 2
    tiles = make_cache(2, nb, hkv, T, dtype=dtype, seed=T + 3)
    rows = rows_twin(tiles)
    q_obs = kvc_synth.queries((w, nb, hq, 128), dtype=dtype, device=DEV, seed=T)
    out = []
    for c in (tiles, rows):
        score = torch.full((nb, hkv, T), float("nan"), device=DEV)
        rng = torch.full((nb, hkv, T), float("nan"), device=DEV)
        kvc.kvc_score(c, 1, q_obs, score, rng, None, ws_tensor(kvc.kvc_score_ws_bytes(c, hq, w)))
        out.append((score, rng))
    torch.cuda.synchronize()
    assert torch.equal(out[0][0], out[1][0]) and torch.equal(out[0][1], out[1][1])
    K, V = slab_np(tiles, 1)
    g = hq // hkv
    ref = oracle.window_score(to_np(q_obs)[:, 1, (hkv - 1) * g:hkv * g], K[1, hkv - 1], T)
    got = out[1][0][1, hkv - 1].double().cpu().numpy()
    assert np.max(np.abs(got - ref) / np.maximum(ref, 1e-30)) <= 1e-5


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("pattern", ["sparse", "dense", "unordered", "ingest"])
def test_compact_from_rows(dtype, pattern):
    """rows -> tiles equals tiles -> tiles bit for bit and the oracle's gather;
    kept = None copies rows [0, n_keep)."""
    say("compact rows", dtype, pattern)
    nb, hkv, T = 2, 4, 1000
    tiles = make_cache(2, nb, hkv, T, dtype=dtype, seed=9)
    rows = rows_twin(tiles)
    g = torch.Generator(device="cpu").manual_seed(1)
    n_keep = {"sparse": 250, "dense": 985, "unordered": 985, "ingest": 1000}[pattern]
    kept = None
    if pattern != "ingest":
        kept = torch.stack([torch.stack([torch.randperm(T, generator=g)[:n_keep].sort().values
                                         for _ in range(hkv)]) for _ in range(nb)])
        if pattern == "unordered":
            kept = kept[..., torch.randperm(n_keep, generator=g)]
        kept = kept.int().contiguous().to(DEV)
        kept[1, 2, 7] = T + 5                                  # out of range -> zero row
    dsts = []
    for src in (tiles, rows):
        d = kvc.Cache.empty(2, nb, hkv, 1024, dtype=dtype, device=DEV)
        d.k.view(torch.int16).fill_(-1)
        d.v.view(torch.int16).fill_(-1)
        kvc.kvc_compact(src, 1, kept, n_keep, d)
        d.t_len = n_keep
        dsts.append(d)
    torch.cuda.synchronize()
    if pattern == "ingest":
        # the tiled source's own rows, re-laid from the rows cache
        assert torch.equal(bits(dsts[1].k[1, :, :, :T]), bits(tiles.k[1, :, :, :T]))
        assert torch.equal(bits(dsts[1].v[1, :, :, :T // 32]), bits(tiles.v[1, :, :, :T // 32]))
        assert torch.equal(bits(dsts[1].v_rows(1)), bits(tiles.v_rows(1)))
        # decode attention over the ingested cache against the oracle on the
        # logical rows of the rows cache
        hq = 4 * hkv
        q = kvc_synth.queries((1, nb, hq, 128), dtype=dtype, device=DEV, seed=77)
        out = torch.empty((1, nb, hq, 128), device=DEV)
        kvc.kvc_decode_attn(dsts[1], q, [1], out, None,
                            ws_tensor(kvc.kvc_decode_attn_ws_bytes(dsts[1], 1, hq)))
        torch.cuda.synchronize()
        Kr = rows.k_rows(1).double().cpu().numpy()
        Vr = rows.v_rows(1).double().cpu().numpy()
        worst = big = 0.0
        for b in range(nb):
            for j in range(hkv):
                ref, _ = oracle.attention(to_np(q[0, b, 4 * j:4 * j + 4]), Kr[b, j], Vr[b, j])
                worst = max(worst, float(np.abs(to_np(out[0, b, 4 * j:4 * j + 4]) - ref).max()))
                big = max(big, float(np.abs(ref).max()))
        say(f"  attention over the ingested cache: max |o - ref| = {worst:.2e}")
        # bf16: 2e-2 absolute; float32: 1e-5 of the largest output
        assert worst <= (2e-2 if dtype == torch.bfloat16 else 1e-5 * big)
        return
    assert torch.equal(bits(dsts[0].k), bits(dsts[1].k))
    assert torch.equal(bits(dsts[0].v), bits(dsts[1].v))
    K, V = slab_np(tiles, 1)
    Kd, Vd = slab_np(dsts[1], 1)
    kp = kept.cpu().numpy()
    for b in range(nb):
        for j in range(hkv):
            ok = kp[b, j] < T
            Kr, Vr = oracle.compact(K[b, j], V[b, j], kp[b, j][ok])
            assert np.array_equal(Kd[b, j][ok], Kr) and np.array_equal(Vd[b, j][ok], Vr)
            assert np.all(Kd[b, j][~ok] == 0) and np.all(Vd[b, j][~ok] == 0)


def test_compact_from_rows_ragged():
    """A batch map on both sides: sequences gathered from rows entries into
    tiled entries; rows past each kept count untouched."""
    say("compact rows ragged")
    hkv, T, n_keep = 4, 900, 300
    tiles = make_cache(2, 3, hkv, T, seed=12)
    rows = rows_twin(tiles)
    lens = [900, 120, 0]
    view = rows.seqs(torch.tensor([2, 0, 1], dtype=torch.int32, device=DEV),
                     torch.tensor(lens, dtype=torch.int32, device=DEV), t_len=T)
    dst = kvc.Cache.empty(2, 4, hkv, 320, device=DEV)
    dst.k.view(torch.int16).fill_(-1)
    dst.v.view(torch.int16).fill_(-1)
    dview = dst.seqs(torch.tensor([3, 1, 0], dtype=torch.int32, device=DEV), None, t_len=n_keep)
    g = torch.Generator(device="cpu").manual_seed(3)
    kept = torch.full((3, hkv, n_keep), -1, dtype=torch.int32)
    for b, Tb in enumerate(lens):
        m = min(Tb, n_keep)
        for j in range(hkv):
            if m:
                kept[b, j, :m] = torch.randperm(Tb, generator=g)[:m].sort().values.int()
    kvc.kvc_compact(view, 0, kept.to(DEV), n_keep, dview)
    torch.cuda.synchronize()
    K, V = slab_np(tiles, 0)
    dst.t_len = n_keep
    Kd, Vd = slab_np(dst, 0)
    src_e, dst_e = [2, 0, 1], [3, 1, 0]
    for b, Tb in enumerate(lens):
        m = min(Tb, n_keep)
        for j in range(hkv):
            ks = kept[b, j, :m].numpy()
            assert np.array_equal(Kd[dst_e[b], j, :m], K[src_e[b], j, ks])
            assert np.array_equal(Vd[dst_e[b], j, :m], V[src_e[b], j, ks])
            assert np.all(np.isnan(Kd[dst_e[b], j, m:]))      # untouched NaN bits
    assert bool((bits(dst.k[:, 2]) == -1).all()) and bool((bits(dst.v[:, 2]) == -1).all())


def test_initial_pass_from_rows_equals_tiles():
    """The Decoder's prompt compression from a rows prompt cache gives the
    tiled decode cache bit for bit as from a tiled prompt cache."""
    say("initial pass rows vs tiles")
    L, leaders, nb, hq, hkv, T = 4, [0, 2], 3, 32, 8, 3000
    ev = dict(K=1000, B=64, N_v=32, w=32, period=64, seed=5)
    tiles = make_cache(2, nb, hkv, T, seed=21)
    rows = rows_twin(tiles)
    q_init = [kvc_synth.queries((ev["w"], nb, hq, 128), device=DEV, seed=30 + i) for i in range(2)]
    res = []
    for prompt in (tiles, rows):
        cache = kvc.Cache.empty(2, nb, hkv, ev["K"] + ev["B"] + ev["period"], device=DEV)
        cache.k.zero_()
        cache.v.zero_()
        dec = Decoder(L, leaders, prompt, cache, hq, evict=ev)
        dec.initial_pass(q_init)
        res.append(dec.cache)
    torch.cuda.synchronize()
    assert res[0].t_len == res[1].t_len == ev["K"] + ev["B"]
    assert torch.equal(bits(res[0].k), bits(res[1].k))
    assert torch.equal(bits(res[0].v), bits(res[1].v))


def test_rows_cache_rejected_by_decode_calls():
    rows = kvc.Cache.empty(1, 1, 2, 64, device=DEV, v_layout="rows", t_len=10)
    q = torch.zeros((1, 1, 8, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((1, 1, 8, 128), device=DEV)
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_decode_attn(rows, q, [0], out, None, ws_tensor(1 << 16))
    assert e.value.status == kvc.KVC_EINVAL
    tiles = kvc.Cache.empty(1, 1, 2, 64, device=DEV, t_len=10)
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_compact(tiles, 0, None, 10, rows)                # rows destination
    assert e.value.status == kvc.KVC_EINVAL


@pytest.mark.parametrize("rank", [16, 32])
def test_dkv_scores_rows_equal_tiles(rank):
    """VASE-DKV scores and the fused range from a rows cache equal the tiled
    form's bit for bit (the same sketch, Gram and leverage arithmetic)."""
    say("dkv rows", rank)
    nb, hkv, T = 2, 4, 2500
    tiles = make_cache(1, nb, hkv, T, seed=31)
    rows = rows_twin(tiles)
    g = kvc_synth.queries((rank, 256), dtype=torch.bfloat16, device=DEV, seed=5)
    out = []
    for c in (tiles, rows):
        sc = torch.full((nb, hkv, T), float("nan"), device=DEV)
        rg = torch.full((nb, hkv, T), float("nan"), device=DEV)
        kvc.kvc_dkv_score(c, 0, g, sc, rg, ws_tensor(kvc.kvc_dkv_ws_bytes(c, rank)))
        out.append((sc, rg))
    torch.cuda.synchronize()
    assert torch.equal(out[0][0], out[1][0]) and torch.equal(out[0][1], out[1][1])


def test_ragged_score_and_range_rows():
    """A batch map and per-sequence lengths on a rows cache: scores (two
    passes: statistics from the keys) and ranges equal the tiled form's."""
    say("ragged score rows")
    hkv, hq, w, T = 4, 20, 16, 1500
    tiles = make_cache(2, 4, hkv, T, seed=41)
    rows = rows_twin(tiles)
    idx = torch.tensor([3, 0, 2], dtype=torch.int32, device=DEV)
    lens = torch.tensor([1500, 40, 777], dtype=torch.int32, device=DEV)
    q_obs = kvc_synth.queries((w, 3, hq, 128), device=DEV, seed=42)
    out = []
    for c in (tiles, rows):
        v = c.seqs(idx, lens, t_len=T)
        sc = torch.full((3, hkv, T), float("nan"), device=DEV)
        rg = torch.full((3, hkv, T), float("nan"), device=DEV)
        kvc.kvc_score(v, 1, q_obs, sc, rg, None, ws_tensor(kvc.kvc_score_ws_bytes(v, hq, w)))
        out.append((sc, rg))
    torch.cuda.synchronize()
    for b, L in enumerate([1500, 40, 777]):
        assert torch.equal(out[0][0][b, :, :L], out[1][0][b, :, :L])
        assert torch.equal(out[0][1][b, :, :L], out[1][1][b, :, :L])
        assert bool(torch.isnan(out[1][1][b, :, L:]).all())     # rows past the length untouched

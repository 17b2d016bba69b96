"""GPU parity of the cross-layer factorisation and selective reconstruction
(kvc_xkv_factor, kvc_xkv_decode_attn) against oracle/xkv.py.

Tolerances (derived from the arithmetic):
* factorisation: the library stores A = X V in bf16 and forms it with V
  rounded to bf16, so a reconstruction carries two bf16 roundings, a relative
  error of about 2 x 2^-9 of the row norms: ||X - A B||_F <= 6e-3 ||X||_F when
  X has rank <= r (the truncation is then exact), and ||X - A B||_F <=
  1.01 opt + 6e-3 ||X||_F with noise, opt = the oracle's truncated-SVD error
  (subspace iteration's excess over the truncation shrinks geometrically;
  12 steps leave ~0.1% on these inputs).
* decode on the oracle's own factors (rounded to the stored types): float32
  rank-space arithmetic against float64, outputs within 1e-3 (the bf16 bar is
  2e-2) and lse within 1e-4; the kept chunk sets equal the oracle's except
  chunks whose oracle score lies within 1e-5 (relative to the largest
  score) of the cutoff, which are counted.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import xkv as oxkv
import kvc_synth
import decode_attention_kvc_amd as kvc
from helpers import ws_tensor, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16_round(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16).double().numpy()


def window_cache(nb, hkv, T, W, k, noise, seed, extra_slots=0):
    """A bf16 cache whose slots [extra_slots, extra_slots + W) hold the W
    layers of one window (NaN bits past T)."""
    layers = kvc_synth.lowrank_layers(nb, hkv, T, W, k, noise=noise, device=DEV, seed=seed)
    c = kvc.Cache.empty(extra_slots + W, nb, hkv, T + 64, device=DEV)
    c.k.view(torch.int16).fill_(-1)
    c.v.view(torch.int16).fill_(-1)
    for l, (K, V) in enumerate(layers):
        c.fill(extra_slots + l, K, V)
    Ks = [K.double().cpu().numpy() for K, _ in layers]
    Vs = [V.double().cpu().numpy() for _, V in layers]
    return c, Ks, Vs


def factor(c, slot0, W, rank, iters=12):
    st = kvc.XkvStore.empty(c.nb, c.n_kv_heads, W, rank, c.t_cap, device=DEV)
    st.t_len = c.t_len
    ws = ws_tensor(kvc.kvc_xkv_factor_ws_bytes(st))
    kvc.kvc_xkv_factor(c, slot0, st, ws, iters=iters, seed=5)
    torch.cuda.synchronize()
    return st


def gpu_recon(st, b, j, l, kv):
    A = (st.ak[b, j] if kv == 0 else st.av_rows(b, j))[:st.t_len].double().cpu().numpy()
    B = (st.bk if kv == 0 else st.bv)[b, j, l * 128:(l + 1) * 128].double().cpu().numpy().T
    return A @ B


FACTOR_CASES = [
    # (nb, hkv, T, W, rank, k, noise)
    (1, 2, 1000, 4, 32, 20, 0.0),
    (2, 1, 1001, 2, 64, 40, 0.0),       # partial last chunk and tile
    (1, 2, 777, 3, 32, 32, 0.0),        # rank exactly r
    (1, 1, 2048, 4, 64, 48, 0.1),       # noisy: truncation error
]


@pytest.mark.parametrize("case", FACTOR_CASES, ids=lambda c: "x".join(map(str, c)))
def test_factor_against_truncated_svd(case):
    nb, hkv, T, W, rank, k, noise = case
    say("xkv factor", case)
    c, Ks, Vs = window_cache(nb, hkv, T, W, k, noise, seed=T + W, extra_slots=1)
    st = factor(c, 1, W, rank)
    worst = 0.0
    for b in range(nb):
        for j in range(hkv):
            for kv, Xs in ((0, Ks), (1, Vs)):
                X = np.hstack([x[b, j] for x in Xs])
                R = np.hstack([gpu_recon(st, b, j, l, kv) for l in range(W)])
                A, Bs = oxkv.clf([x[b, j] for x in Xs], rank)
                opt = np.linalg.norm(X - np.hstack([A @ B for B in Bs]))
                err = np.linalg.norm(X - R)
                nx = np.linalg.norm(X)
                worst = max(worst, (err - opt) / nx)
                assert err <= 1.01 * opt + 6e-3 * nx, (b, j, kv, err / nx, opt / nx)
            # bases: orthonormal columns
            for basis in (st.bk, st.bv):
                Vb = basis[b, j].double().cpu().numpy()
                assert np.abs(Vb.T @ Vb - np.eye(rank)).max() <= 1e-4
            # landmarks: chunk means of the stored key basis
            A = st.ak[b, j, :T].float()
            n = (T + 7) // 8
            pad = torch.zeros((n * 8 - T, rank), device=DEV)
            sums = torch.cat([A, pad]).view(n, 8, rank).sum(1)
            cnt = torch.tensor([min(8, T - 8 * i) for i in range(n)], device=DEV, dtype=torch.float32)
            want = (sums / cnt[:, None]).to(torch.bfloat16).float()
            got = st.lk[b, j, :n].float()
            assert torch.allclose(got, want, rtol=2 ** -7, atol=1e-6)
    say(f"  worst (err - opt) / ||X||: {worst:.2e}")


def oracle_store(Ks, Vs, rank, t_cap):
    """The oracle's factors, rounded to the stored types, as an XkvStore."""
    nb, hkv, T, _ = Ks[0].shape
    W = len(Ks)
    st = kvc.XkvStore.empty(nb, hkv, W, rank, t_cap, device=DEV, t_len=T)
    st.lk.zero_()
    fac = {}
    for b in range(nb):
        for j in range(hkv):
            AK, BK = oxkv.clf([x[b, j] for x in Ks], rank)
            AV, BV = oxkv.clf([x[b, j] for x in Vs], rank)
            AKr, AVr = bf16_round(AK), bf16_round(AV)
            L = bf16_round(oxkv.landmarks(AKr, 8))
            BKf = [np.asarray(B, dtype=np.float32).astype(np.float64) for B in BK]
            BVf = [np.asarray(B, dtype=np.float32).astype(np.float64) for B in BV]
            st.ak[b, j, :T] = torch.as_tensor(AKr, dtype=torch.bfloat16)
            st.set_av_rows(b, j, torch.as_tensor(AVr, dtype=torch.bfloat16, device=DEV))
            st.lk[b, j, :len(L)] = torch.as_tensor(L, dtype=torch.bfloat16)
            st.bk[b, j] = torch.as_tensor(np.vstack([B.T for B in BKf]), dtype=torch.float32)
            st.bv[b, j] = torch.as_tensor(np.vstack([B.T for B in BVf]), dtype=torch.float32)
            fac[(b, j)] = (AKr, AVr, L, BKf, BVf)
    return st, fac


DECODE_CASES = [
    # (nb, hkv, hq, T, W, rank, n_select)
    (2, 2, 8, 1000, 4, 32, 40),
    (1, 4, 32, 3001, 2, 64, 128),       # partial last chunk
    (1, 2, 16, 600, 4, 64, 200),        # every chunk kept (75 chunks)
    (2, 1, 4, 4096, 3, 32, 64),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "x".join(map(str, c)))
def test_decode_on_oracle_factors(case):
    nb, hkv, hq, T, W, rank, n_select = case
    say("xkv decode", case)
    layers = kvc_synth.lowrank_layers(nb, hkv, T, W, 24, noise=0.2, device="cpu", seed=T)
    Ks = [K.double().numpy() for K, _ in layers]
    Vs = [V.double().numpy() for _, V in layers]
    st, fac = oracle_store(Ks, Vs, rank, T + 64)
    g = hq // hkv
    q = kvc_synth.queries((nb, hq, 128), device=DEV, seed=T + 1)
    qn = to_np(q)
    ws = ws_tensor(kvc.kvc_xkv_decode_ws_bytes(st, hq, n_select))
    flips = 0
    for layer in range(W):
        out = torch.full((nb, hq, 128), float("nan"), device=DEV)
        lse = torch.full((nb, hq), float("nan"), device=DEV)
        sel = torch.full((nb, hkv, n_select), -7, dtype=torch.int32, device=DEV)
        kvc.kvc_xkv_decode_attn(st, layer, q, out, lse, n_select=n_select, selected=sel, ws=ws)
        torch.cuda.synchronize()
        o, l, s = to_np(out), to_np(lse), sel.cpu().numpy()
        nch = (T + 7) // 8
        for b in range(nb):
            for j in range(hkv):
                AK, AV, L, BK, BV = fac[(b, j)]
                qh = qn[b, j * g:(j + 1) * g]
                ro, rl, kept = oxkv.sr_attention(qh, AK, AV, BK[layer], BV[layer], L, 8, n_select)
                k = len(kept)
                assert np.all(s[b, j, k:] == -1)
                got = s[b, j, :k]
                if not np.array_equal(got, kept):
                    sc = oxkv.chunk_scores(qh, BK[layer], L)
                    cut = np.sort(sc)[::-1][k - 1]
                    for ch in set(got.tolist()) ^ set(kept.tolist()):
                        assert abs(sc[ch] - cut) <= 1e-5 * np.abs(sc).max(), (layer, b, j, ch)
                    flips += 1
                    continue
                assert np.abs(o[b, j * g:(j + 1) * g] - ro).max() <= 1e-3
                assert np.abs(l[b, j * g:(j + 1) * g] - rl).max() <= 1e-4
    say(f"  slabs with a flipped chunk inside the band: {flips}")


def test_decode_merges_a_second_part():
    """Rows appended after the factorisation: attended by kvc_decode_attn over
    a small tail cache and merged; the oracle merges its own two parts."""
    say("xkv decode merge")
    nb, hkv, hq, T, W, rank, n_sel, tail = 1, 2, 8, 900, 2, 32, 30, 45
    layers = kvc_synth.lowrank_layers(nb, hkv, T, W, 16, noise=0.1, device="cpu", seed=4)
    Ks = [K.double().numpy() for K, _ in layers]
    Vs = [V.double().numpy() for _, V in layers]
    st, fac = oracle_store(Ks, Vs, rank, T)
    tc = kvc.Cache.empty(W, nb, hkv, tail + 19, device=DEV)
    Kt, Vt, _, _ = kvc_synth.kv_slot(nb, hkv, tail, device=DEV, seed=9)
    tc.fill(1, Kt, Vt)
    q = kvc_synth.queries((1, nb, hq, 128), device=DEV, seed=8)
    o_t = torch.empty((1, nb, hq, 128), device=DEV)
    l_t = torch.empty((1, nb, hq), device=DEV)
    kvc.kvc_decode_attn(tc, q, [1], o_t, l_t, ws_tensor(kvc.kvc_decode_attn_ws_bytes(tc, 1, hq)))
    out = torch.empty((nb, hq, 128), device=DEV)
    lse = torch.empty((nb, hq), device=DEV)
    kvc.kvc_xkv_decode_attn(st, 1, q[0], out, lse, n_select=n_sel, o_in=o_t[0], lse_in=l_t[0],
                            ws=ws_tensor(kvc.kvc_xkv_decode_ws_bytes(st, hq, n_sel)))
    torch.cuda.synchronize()
    g = hq // hkv
    qn = to_np(q[0])
    Ktn, Vtn = Kt.double().cpu().numpy(), Vt.double().cpu().numpy()
    for j in range(hkv):
        AK, AV, L, BK, BV = fac[(0, j)]
        qh = qn[0, j * g:(j + 1) * g]
        o1, l1, _ = oxkv.sr_attention(qh, AK, AV, BK[1], BV[1], L, 8, n_sel)
        o2, l2 = oracle.attention(qh, Ktn[0, j], Vtn[0, j])
        ro, rl = oxkv.merge_attention(o1, l1, o2, l2)
        assert np.abs(to_np(out[0, j * g:(j + 1) * g]) - ro).max() <= 1e-3
        assert np.abs(to_np(lse[0, j * g:(j + 1) * g]) - rl).max() <= 1e-4


def test_factor_then_decode_end_to_end():
    """Exact rank-k layers, every chunk kept: the library's factorisation
    followed by its decode equals plain attention over the original rows, up
    to the bf16 storage of the bases."""
    say("xkv end to end")
    nb, hkv, hq, T, W, rank = 1, 2, 8, 700, 4, 32
    c, Ks, Vs = window_cache(nb, hkv, T, W, 16, 0.0, seed=12)
    st = factor(c, 0, W, rank)
    q = kvc_synth.queries((nb, hq, 128), device=DEV, seed=13)
    g = hq // hkv
    qn = to_np(q)
    worst = 0.0
    ws = ws_tensor(kvc.kvc_xkv_decode_ws_bytes(st, hq, 512))
    for layer in range(W):
        out = torch.empty((nb, hq, 128), device=DEV)
        kvc.kvc_xkv_decode_attn(st, layer, q, out, n_select=512, ws=ws)
        torch.cuda.synchronize()
        for j in range(hkv):
            ro, _ = oracle.attention(qn[0, j * g:(j + 1) * g], Ks[layer][0, j], Vs[layer][0, j])
            worst = max(worst, np.abs(to_np(out[0, j * g:(j + 1) * g]) - ro).max())
    say(f"  max |o - attention over the original rows| = {worst:.2e}")
    assert worst <= 2e-2


def test_decode_full_size_sampled():
    """The launch shape of the bench's cross-layer leg (batch 16, 8 KV heads,
    32 query heads, 32768 rows, a window of 4 layers at rank 64, 256 of 4096
    chunks kept, a tail part merged in): seeded store contents and tail
    outputs are the inputs, and sampled (batch entry, KV head) pairs are
    checked against the oracle's selective reconstruction and merge."""
    nb, hkv, hq, T, W, R, n_sel = 16, 8, 32, 32768, 4, 64, 256
    g = hq // hkv
    say("xkv decode full size")
    st = kvc.XkvStore.empty(nb, hkv, W, R, T, device=DEV, t_len=T)
    st.ak.copy_(kvc_synth.queries(st.ak.shape, device=DEV, seed=101))
    st.av.copy_(kvc_synth.queries(st.av.shape, device=DEV, seed=102))
    st.lk.copy_(kvc_synth.queries(st.lk.shape, device=DEV, seed=103))
    st.bk.copy_(kvc_synth.queries(st.bk.shape, dtype=torch.float32, device=DEV, seed=104) * 128 ** -0.5)
    st.bv.copy_(kvc_synth.queries(st.bv.shape, dtype=torch.float32, device=DEV, seed=105) * 128 ** -0.5)
    q = kvc_synth.queries((nb, hq, 128), device=DEV, seed=106)
    o_in = kvc_synth.queries((nb, hq, 128), dtype=torch.float32, device=DEV, seed=107)
    lse_in = kvc_synth.queries((nb, hq), dtype=torch.float32, device=DEV, seed=108) + 8.0
    layer = 2
    out = torch.full((nb, hq, 128), float("nan"), device=DEV)
    lse = torch.full((nb, hq), float("nan"), device=DEV)
    sel = torch.full((nb, hkv, n_sel), -7, dtype=torch.int32, device=DEV)
    ws = ws_tensor(kvc.kvc_xkv_decode_ws_bytes(st, hq, n_sel))
    kvc.kvc_xkv_decode_attn(st, layer, q, out, lse, n_select=n_sel, o_in=o_in, lse_in=lse_in,
                            selected=sel, ws=ws)
    torch.cuda.synchronize()
    nch = T // 8
    flips = 0
    for (b, j) in [(0, 0), (7, 3), (15, 7), (9, 5)]:
        AK = st.ak[b, j, :T].double().cpu().numpy()
        AV = st.av_rows(b, j)[:T].double().cpu().numpy()
        L = st.lk[b, j, :nch].double().cpu().numpy()
        BK = st.bk[b, j, layer * 128:(layer + 1) * 128].double().cpu().numpy().T
        BV = st.bv[b, j, layer * 128:(layer + 1) * 128].double().cpu().numpy().T
        qh = to_np(q[b, j * g:(j + 1) * g])
        o1, l1, kept = oxkv.sr_attention(qh, AK, AV, BK, BV, L, 8, n_sel)
        ro, rl = oxkv.merge_attention(o1, l1, to_np(o_in[b, j * g:(j + 1) * g]),
                                      to_np(lse_in[b, j * g:(j + 1) * g]))
        got = sel[b, j].cpu().numpy()
        if not np.array_equal(got, kept):
            sc = oxkv.chunk_scores(qh, BK, L)
            cut = np.sort(sc)[::-1][n_sel - 1]
            for ch in set(got.tolist()) ^ set(kept.tolist()):
                assert abs(sc[ch] - cut) <= 1e-5 * np.abs(sc).max(), (b, j, ch)
            flips += 1
            continue
        assert np.abs(to_np(out[b, j * g:(j + 1) * g]) - ro).max() <= 1e-3, (b, j)
        assert np.abs(to_np(lse[b, j * g:(j + 1) * g]) - rl).max() <= 1e-4, (b, j)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    say(f"  sampled pairs with a flipped chunk inside the band: {flips}")


def random_store(nb, hkv, T, W, R, seed):
    """Seeded N(0, 1) store contents (the decode needs no factorisation)."""
    st = kvc.XkvStore.empty(nb, hkv, W, R, T, device=DEV, t_len=T)
    st.ak.copy_(kvc_synth.queries(st.ak.shape, device=DEV, seed=seed))
    st.av.copy_(kvc_synth.queries(st.av.shape, device=DEV, seed=seed + 1))
    st.lk.copy_(kvc_synth.queries(st.lk.shape, device=DEV, seed=seed + 2))
    st.bk.copy_(kvc_synth.queries(st.bk.shape, dtype=torch.float32, device=DEV, seed=seed + 3)
                * 128 ** -0.5)
    st.bv.copy_(kvc_synth.queries(st.bv.shape, dtype=torch.float32, device=DEV, seed=seed + 4)
                * 128 ** -0.5)
    return st


def check_pairs(st, q, out, lse, sel, layer, n_sel, pairs, exact_sel=False):
    """Sampled (b, j) pairs against the oracle's selective reconstruction;
    chunks kept by one side only must sit within 1e-5 of the cutoff score
    unless exact_sel.  Returns the number of pairs with such a flip."""
    T, hkv = st.t_len, st.n_kv_heads
    g = q.shape[1] // hkv
    nch = (T + 7) // 8
    flips = 0
    for (b, j) in pairs:
        AK = st.ak[b, j, :T].double().cpu().numpy()
        AV = st.av_rows(b, j)[:T].double().cpu().numpy()
        L = st.lk[b, j, :nch].double().cpu().numpy()
        BK = st.bk[b, j, layer * 128:(layer + 1) * 128].double().cpu().numpy().T
        BV = st.bv[b, j, layer * 128:(layer + 1) * 128].double().cpu().numpy().T
        qh = to_np(q[b, j * g:(j + 1) * g])
        ro, rl, kept = oxkv.sr_attention(qh, AK, AV, BK, BV, L, 8, n_sel)
        got = sel[b, j].cpu().numpy()
        k = len(kept)
        assert np.all(got[k:] == -1)
        if not np.array_equal(got[:k], kept):
            assert not exact_sel, (b, j)
            sc = oxkv.chunk_scores(qh, BK, L)
            cut = np.sort(sc)[::-1][k - 1]
            for ch in set(got[:k].tolist()) ^ set(kept.tolist()):
                assert abs(sc[ch] - cut) <= 1e-5 * np.abs(sc).max(), (b, j, ch)
            flips += 1
            continue
        assert np.abs(to_np(out[b, j * g:(j + 1) * g]) - ro).max() <= 1e-3, (b, j)
        assert np.abs(to_np(lse[b, j * g:(j + 1) * g]) - rl).max() <= 1e-4, (b, j)
    return flips


def run_decode(st, q, layer, n_sel):
    nb, hq = q.shape[0], q.shape[1]
    out = torch.full((nb, hq, 128), float("nan"), device=DEV)
    lse = torch.full((nb, hq), float("nan"), device=DEV)
    sel = torch.full((nb, st.n_kv_heads, n_sel), -7, dtype=torch.int32, device=DEV)
    ws = ws_tensor(kvc.kvc_xkv_decode_ws_bytes(st, hq, n_sel))
    kvc.kvc_xkv_decode_attn(st, layer, q, out, lse, n_select=n_sel, selected=sel, ws=ws)
    torch.cuda.synchronize()
    return out, lse, sel


def test_decode_long_store_uses_the_workspace_path():
    """170000 rows at rank 64 (21250 chunk keys, more than one workgroup's
    LDS holds beside the rest): the top-k reads the chunk keys from the
    workspace instead of LDS, against the oracle."""
    say("xkv decode, long store")
    nb, hkv, hq, T, W, R, n_sel = 1, 2, 8, 170000, 2, 64, 64
    st = random_store(nb, hkv, T, W, R, seed=301)
    q = kvc_synth.queries((nb, hq, 128), device=DEV, seed=306)
    out, lse, sel = run_decode(st, q, 1, n_sel)
    flips = check_pairs(st, q, out, lse, sel, 1, n_sel, [(0, 0), (0, 1)])
    say(f"  pairs with a flipped chunk inside the band: {flips}")


@pytest.mark.parametrize("levels", [1, 3])
def test_decode_selection_ties(levels):
    """Landmarks that take only `levels` distinct rows, so most chunk scores
    tie exactly: the kept chunks must be the oracle's (ties to the lower
    chunk), with the keys in LDS (4100 chunks) and read from the workspace
    (21250)."""
    for T, R in [(32800, 64), (170000, 64)]:
        say("xkv selection ties", levels, T)
        nb, hkv, hq, W, n_sel = 1, 2, 8, 2, 200
        st = random_store(nb, hkv, T, W, R, seed=400 + levels)
        nch = (T + 7) // 8
        pick = torch.randint(0, levels, (nb, hkv, nch), generator=torch.Generator().manual_seed(levels))
        rows = kvc_synth.queries((levels, R), device=DEV, seed=410 + levels).to(torch.bfloat16)
        st.lk[:, :, :nch] = rows[pick.to(DEV)]
        q = kvc_synth.queries((nb, hq, 128), device=DEV, seed=420 + levels)
        out, lse, sel = run_decode(st, q, 0, n_sel)
        check_pairs(st, q, out, lse, sel, 0, n_sel, [(0, 0), (0, 1)], exact_sel=True)


EDGE_CASES = [
    # (nb, hkv, hq, T, W, R, n_select)
    (1, 1, 1, 1, 2, 32, 1),          # one row, one head
    (1, 2, 6, 7, 3, 64, 1),          # one partial chunk
    (2, 1, 3, 9, 2, 32, 1),          # two chunks, keep one (g = 3)
    (1, 2, 10, 17, 4, 64, 2),        # g = 5, partial last chunk kept or not
    (1, 1, 7, 1001, 2, 32, 126),     # g = 7, ~all but a few chunks
    (1, 2, 16, 4100, 2, 64, 513),    # g = 8, more kept chunks than the old 16384-row cap
    (3, 2, 4, 260, 1, 64, 40),       # g = 2, window of one layer
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=lambda c: "x".join(map(str, c)))
def test_decode_edge_shapes(case):
    """Small, ragged and odd shapes of the decode (one row, one
    partial chunk, odd head groups up to 8, every chunk or all but a few kept)
    against the oracle for every (b, j) and every layer of the window."""
    nb, hkv, hq, T, W, R, n_sel = case
    say("xkv decode edge", case)
    st = random_store(nb, hkv, T, W, R, seed=500 + T)
    q = kvc_synth.queries((nb, hq, 128), device=DEV, seed=600 + T)
    flips = 0
    for layer in range(W):
        out, lse, sel = run_decode(st, q, layer, n_sel)
        pairs = [(b, j) for b in range(nb) for j in range(hkv)]
        flips += check_pairs(st, q, out, lse, sel, layer, n_sel, pairs)
    say(f"  pairs with a flipped chunk inside the band: {flips}")


def test_decode_one_workspace_for_two_store_shapes():
    """One zeroed workspace, sized for the larger store, serves calls on two
    stores of different shapes in turn (40 and 3 (b, j), so seven and eight
    workgroups per (b, j)): the arrival counters sit at the workspace's start
    and every call leaves them zero, so each call merges its own splits."""
    say("xkv decode, one workspace for two shapes")
    big = random_store(5, 8, 2000, 2, 64, seed=700)
    small = random_store(1, 3, 900, 3, 32, seed=710)
    q_big = kvc_synth.queries((5, 32, 128), device=DEV, seed=720)
    q_small = kvc_synth.queries((1, 6, 128), device=DEV, seed=721)
    n_sel = 40
    ws = ws_tensor(max(kvc.kvc_xkv_decode_ws_bytes(big, 32, n_sel),
                       kvc.kvc_xkv_decode_ws_bytes(small, 6, n_sel)))
    flips = 0
    for it, (st, q, layer) in enumerate([(big, q_big, 0), (small, q_small, 2), (big, q_big, 1),
                                         (small, q_small, 0), (big, q_big, 1)]):
        nb, hq = q.shape[0], q.shape[1]
        out = torch.full((nb, hq, 128), float("nan"), device=DEV)
        lse = torch.full((nb, hq), float("nan"), device=DEV)
        sel = torch.full((nb, st.n_kv_heads, n_sel), -7, dtype=torch.int32, device=DEV)
        kvc.kvc_xkv_decode_attn(st, layer, q, out, lse, n_select=n_sel, selected=sel, ws=ws)
        torch.cuda.synchronize()
        pairs = [(b, j) for b in range(nb) for j in range(st.n_kv_heads)]
        flips += check_pairs(st, q, out, lse, sel, layer, n_sel, pairs)
        assert torch.isfinite(out).all()
    assert int(ws[:256].view(torch.int32).abs().sum()) == 0       # counters left at zero
    say(f"  pairs with a flipped chunk inside the band: {flips}")

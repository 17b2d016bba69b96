"""GPU parity of the VASE-DKV scoring path (kvc_gaussian_bf16, kvc_dkv_score)
against oracle/dkv.py, through the C ABI.

Tolerance of the scores (derived from the arithmetic, not fitted): Y = [K|V] G
is accumulated in float32 from exact bf16 products over 256 terms, so each
entry carries a relative error of a few 2^-24; the Gram matrix, its
factorisation, the inverse factor W and the quadratic form ||y_t W||^2 are
float64 and add nothing at this scale.  Bound, elementwise:
|l - l_ref| <= 1e-6 l_ref + 1e-7 max(l_ref) (helpers.dkv_tolerance; measured:
at most 3.4e-7 of the row's own score).  Kept sets follow the window-score
rule: a row kept by one side only must lie within 1e-6 (relative) of the
oracle's sampling cutoff (a tie, counted); any other difference fails.  The
sum of the scores must equal rank(Y) to 1e-4 relative."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import dkv as odkv
import kvc_synth
import decode_attention_kvc_amd as kvc
from helpers import make_cache, slab_np, ws_tensor, dkv_tolerance, band_compare

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def sketch_matrix(rank, seed):
    """G as the library takes it: bf16 [rank][256]."""
    return kvc_synth.queries((rank, 256), dtype=torch.bfloat16, device=DEV, seed=seed)


def g_for_oracle(g):
    return g.double().cpu().numpy().T           # [256][rank]


@pytest.mark.parametrize("n,seed,c1,c2", [(100003, 7, 3, 0xFFFFFFFF), (64, 0, 0, 0),
                                          (4097, 2**40 + 5, 17, 9)])
def test_gaussian_bit_exact(n, seed, c1, c2):
    say("gaussian", n, seed, c1, c2)
    out = torch.zeros(n + 1, dtype=torch.bfloat16, device=DEV)
    out[n] = 12.5                                     # sentinel past the end
    kvc.kvc_gaussian_bf16(n, seed, c1, c2, out)
    torch.cuda.synchronize()
    got = out[:n].view(torch.int16).cpu().numpy().astype(np.uint16)
    want = odkv.gaussian_bf16(n, seed, c1, c2)
    mism = int((got != want).sum())
    say(f"  mismatching words: {mism} of {n}")
    assert mism == 0
    assert out[n].item() == 12.5


DKV_CASES = [
    # (nb, hkv, T, rank)
    (1, 2, 100, 16),
    (1, 2, 100, 32),
    (2, 8, 1000, 32),
    (1, 8, 4097, 32),          # ragged last tile
    (3, 2, 33, 16),
    (1, 1, 20, 32),            # fewer rows than sketch columns: dropped pivots
    (1, 4, 8448, 32),
]


def check_scores(got, ref, K, V, G):
    err = np.abs(got - ref)
    bound = dkv_tolerance(ref)
    rel = float(np.max(err / np.maximum(ref, 1e-30)))
    say(f"    max |err| / max(ref) {err.max() / ref.max():.2e}, max |err| / ref {rel:.2e}")
    assert np.all(err <= bound), (float(err.max()), bound)
    return float(err.max() / ref.max())


@pytest.mark.parametrize("case", DKV_CASES, ids=lambda c: "x".join(map(str, c)))
def test_dkv_score_matches_oracle(case):
    nb, hkv, T, rank = case
    say("dkv score", case)
    cache = make_cache(2, nb, hkv, T, seed=T + rank)
    g = sketch_matrix(rank, seed=T)
    score = torch.full((nb, hkv, T), float("nan"), device=DEV)
    rng = torch.full((nb, hkv, T), float("nan"), device=DEV)
    ws = ws_tensor(kvc.kvc_dkv_ws_bytes(cache, rank))
    kvc.kvc_dkv_score(cache, 1, g, score, rng, ws)
    torch.cuda.synchronize()
    K, V = slab_np(cache, 1)
    G = g_for_oracle(g)
    worst = 0.0
    for b in range(nb):
        for j in range(hkv):
            ref = odkv.dkv_score(K[b, j], V[b, j], G)
            got = score[b, j].double().cpu().numpy()
            worst = max(worst, check_scores(got, ref, K[b, j], V[b, j], G))
            rk = min(T, rank)
            assert got.sum() == pytest.approx(rk, rel=1e-4)
            assert np.array_equal(rng[b, j].cpu().numpy(),
                                  oracle.value_range(V[b, j]).astype(np.float32))
    say(f"  max error / max score: {worst:.2e}")


def test_dkv_rank_deficient_rows():
    # every row of the slab is one of three (K, V) rows: rank 3 < 16
    say("dkv rank deficient")
    nb, hkv, T, rank = 1, 2, 200, 16
    cache = make_cache(1, nb, hkv, T, seed=3)
    K = cache.k_rows(0)
    V = cache.v_rows(0)
    idx = torch.arange(T, device=DEV) % 3
    cache.fill(0, K[:, :, idx].contiguous(), V[:, :, idx].contiguous())
    g = sketch_matrix(rank, seed=11)
    score = torch.empty((nb, hkv, T), device=DEV)
    ws = ws_tensor(kvc.kvc_dkv_ws_bytes(cache, rank))
    kvc.kvc_dkv_score(cache, 0, g, score, None, ws)
    torch.cuda.synchronize()
    Kn, Vn = slab_np(cache, 0)
    for j in range(hkv):
        got = score[0, j].double().cpu().numpy()
        ref = odkv.dkv_score(Kn[0, j], Vn[0, j], g_for_oracle(g))
        assert got.sum() == pytest.approx(3.0, rel=1e-4)
        check_scores(got, ref, Kn[0, j], Vn[0, j], g_for_oracle(g))


def test_dkv_workspace_reuse_and_determinism():
    say("dkv reuse")
    cache = make_cache(1, 2, 8, 3000, seed=5)
    g = sketch_matrix(32, seed=1)
    ws = ws_tensor(kvc.kvc_dkv_ws_bytes(cache, 32))
    s1 = torch.empty((2, 8, 3000), device=DEV)
    s2 = torch.empty_like(s1)
    kvc.kvc_dkv_score(cache, 0, g, s1, None, ws)
    cache.t_len = 1700                       # a shorter slab in the same workspace
    s3 = torch.empty((2, 8, 1700), device=DEV)
    kvc.kvc_dkv_score(cache, 0, g, s3, None, ws)
    cache.t_len = 3000
    kvc.kvc_dkv_score(cache, 0, g, s2, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    K, V = slab_np(cache, 0)
    ref = odkv.dkv_score(K[1, 3, :1700], V[1, 3, :1700], g_for_oracle(g))
    check_scores(s3[1, 3].double().cpu().numpy(), ref, K[1, 3, :1700], V[1, 3, :1700],
                 g_for_oracle(g))


def test_dkv_kept_sets_match_oracle():
    """End to end: DKV scores -> VASE selection, against the oracle's own
    scores and selection.  Rows within 1e-6 of the sampling cutoff may flip
    (ties, counted); nothing else may."""
    say("dkv select")
    nb, hkv, T, rank = 1, 8, 4352, 32
    Kb, B, Nv = 4096, 128, 64
    cache = make_cache(1, nb, hkv, T, seed=9)
    g = sketch_matrix(rank, seed=21)
    score = torch.empty((nb, hkv, T), device=DEV)
    rng = torch.empty((nb, hkv, T), device=DEV)
    kvc.kvc_dkv_score(cache, 0, g, score, rng, ws_tensor(kvc.kvc_dkv_ws_bytes(cache, rank)))
    kept = torch.empty((nb, hkv, Kb + B), dtype=torch.int32, device=DEV)
    kvc.kvc_select(score, rng, nb, hkv, T, Kb, B, Nv, 99, 3, kept,
                   ws_tensor(kvc.kvc_select_ws_bytes(nb, hkv, T)))
    torch.cuda.synchronize()
    K, V = slab_np(cache, 0)
    ties = 0
    for j in range(hkv):
        sc = odkv.dkv_score(K[0, j], V[0, j], g_for_oracle(g))
        d = oracle.select_detail(sc, oracle.value_range(V[0, j]), T, Kb, B, Nv, 99, 3, 0, j)
        t, bad = band_compare(kept[0, j].cpu().numpy(), d, rel=1e-6)
        assert bad == 0, j
        ties += t
    say(f"  ties within 1e-6 of the cutoff: {ties}")


def test_decoder_dkv_initial_pass():
    """The decode loop's VASE-DKV pass: G drawn by the library per leader
    (key seed + pass, counter (pair, leader layer, 0xFFFFFFFF)), scores,
    selection and compaction; the oracle regenerates G from the same
    definition and selects on its own scores."""
    from decode_attention_kvc_amd.loop import Decoder
    say("decoder dkv initial pass")
    L, leaders, nb, hq, hkv, T0 = 4, [0, 2], 2, 16, 4, 3000
    ev = dict(K=1024, B=64, N_v=32, w=32, period=64, seed=11, scoring="dkv", rank=32)
    big = make_cache(len(leaders), nb, hkv, T0, seed=4)
    pre = [slab_np(big, s) for s in range(len(leaders))]
    cap = ev["K"] + ev["B"] + ev["period"]
    cache = kvc.Cache.empty(len(leaders), nb, hkv, cap, device=DEV)
    dec = Decoder(L, leaders, big, cache, hq, evict=ev)
    dec.initial_pass()
    torch.cuda.synchronize()
    assert dec.cache.t_len == ev["K"] + ev["B"]
    flips = 0
    for s, leader in enumerate(leaders):
        G = odkv.bf16_bits_to_f64(odkv.gaussian_bf16(32 * 256, ev["seed"], leader, 0xFFFFFFFF))
        G = G.reshape(32, 256).T
        K0, V0 = pre[s]
        K1, V1 = slab_np(dec.cache, s)
        for b in range(nb):
            for j in range(hkv):
                sc = odkv.dkv_score(K0[b, j], V0[b, j], G)
                d = oracle.select_detail(sc, oracle.value_range(V0[b, j]), T0, ev["K"], ev["B"],
                                         ev["N_v"], ev["seed"], leader, b, j)
                rows = {K0[b, j, t].tobytes(): t for t in range(T0)}
                kept = np.array([rows[K1[b, j, i].tobytes()] for i in range(len(K1[b, j]))])
                assert np.all(np.diff(kept) > 0)
                assert np.array_equal(V1[b, j], V0[b, j, kept])
                t, bad = band_compare(kept, d, rel=1e-6)
                assert bad == 0, (s, b, j)
                flips += t
    say(f"  ties within 1e-6 of the cutoff: {flips}")

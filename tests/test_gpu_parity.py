"""GPU parity of every libkvc entry point against the float64 oracle.

Tolerances: bfloat16 caches max|o - o_ref| <= 2e-2 (the stated bar; the
measured error is far below it), float32 caches max|o - o_ref| <=
1e-5 * max|o_ref|.  Value ranges and compaction are bit-exact.  Kept sets
are exact except rows whose oracle key lies within 1e-6 (relative) of the
oracle's cutoff; those are counted as ties and reported."""
import math
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


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def oracle_decode(cache, q, q_slot):
    """Oracle outputs for q [nq][nb][Hq][d] over the cache's slots."""
    nq, nb, hq, d = q.shape
    qn = to_np(q)
    Ks, Vs = {}, {}
    for s in set(int(x) for x in q_slot):
        Ks[s], Vs[s] = slab_np(cache, s)
    K = [Ks.get(s) for s in range(cache.n_slots)]
    V = [Vs.get(s) for s in range(cache.n_slots)]
    return oracle.decode_attention(qn, K, V, q_slot, cache.n_kv_heads, cache.t_len)


def run_decode(cache, q, q_slot, with_lse=True, **kw):
    nq, nb, hq, d = q.shape
    out = torch.full((nq, nb, hq, d), float("nan"), device=DEV)
    lse = torch.full((nq, nb, hq), float("nan"), device=DEV) if with_lse else None
    ws = ws_tensor(kvc.kvc_decode_attn_ws_bytes(cache, nq, hq))
    kvc.kvc_decode_attn(cache, q, q_slot, out, lse, ws, **kw)
    torch.cuda.synchronize()
    return out, lse


ATTN_CASES = [
    # (nb, hq, hkv, T, nq, q_slot)
    (1, 8, 2, 1, 1, [0]),
    (1, 8, 2, 31, 1, [0]),
    (2, 32, 8, 33, 1, [0]),
    (1, 32, 8, 64, 1, [1]),
    (1, 40, 8, 1000, 1, [0]),
    (3, 16, 4, 4097, 1, [1]),
    (1, 32, 8, 2500, 4, [0, 0, 0, 0]),        # grouped: 16 query rows
    (2, 40, 8, 777, 2, [1, 1]),               # grouped, g = 5
    (1, 64, 8, 900, 8, [0] * 8),              # 64 query rows (four column blocks)
    (1, 16, 8, 300, 3, [0, 0, 0]),            # 6 rows
    (2, 32, 8, 1500, 4, [0, 1, 0, 1]),        # two slots in one call
    (1, 8, 8, 200, 20, [0] * 20),             # 20 layers, MHA: two launches
    # 128-255 slabs: two splits per slab
    (16, 32, 8, 1031, 1, [0]),
    (33, 16, 4, 300, 1, [1]),                 # 132 slabs: part of the last group idle
    (16, 32, 8, 500, 4, [0, 0, 0, 0]),        # grouped, 16 rows
    (16, 32, 8, 400, 8, [1] * 8),             # 32 rows (two column blocks)
    (256, 32, 8, 300, 1, [0]),                # 2048 slabs: one split each, no merge launch
    (1, 64, 1, 262145, 1, [1]),               # one 256K-row slab, g = 64: the split cap
]


def test_decode_attn_one_workspace_for_many_shapes():
    """One zeroed workspace serves attention calls of several shapes in turn:
    launches whose last workgroup per slab merges (2 to 32 splits per slab)
    and launches merged by the second kernel (16 query rows at 32 splits),
    different slab counts and lengths.  Each output is checked against the
    oracle, and the workspace's counter head is zero after every call."""
    shapes = [
        # (nb, hq, hkv, T, nq, q_slot)
        (1, 32, 8, 33000, 1, [1]),          # 8 slabs x 32 splits, 4 rows: merged in the last workgroup
        (16, 32, 8, 8400, 1, [0]),          # 128 slabs x 2 splits
        (1, 32, 8, 33000, 4, [0] * 4),      # 16 rows at 32 splits: the merge kernel
        (4, 40, 8, 9000, 1, [1]),           # 32 slabs x 8 splits, g = 5
        (8, 32, 8, 4300, 1, [0]),           # 64 slabs x 4 splits
        (1, 32, 8, 33000, 1, [0]),
    ]
    caches = {}
    need = 0
    for (nb, hq, hkv, T, nq, _) in shapes:
        if (nb, hkv, T) not in caches:
            caches[(nb, hkv, T)] = make_cache(2, nb, hkv, T, seed=nb + T)
        need = max(need, kvc.kvc_decode_attn_ws_bytes(caches[(nb, hkv, T)], nq, hq))
    ws = ws_tensor(need)
    for i, (nb, hq, hkv, T, nq, q_slot) in enumerate(shapes):
        say("attention, shared workspace", nb, hq, hkv, T, nq)
        cache = caches[(nb, hkv, T)]
        q = kvc_synth.queries((nq, nb, hq, 128), device=DEV, seed=50 + i)
        out = torch.full((nq, nb, hq, 128), float("nan"), device=DEV)
        lse = torch.full((nq, nb, hq), float("nan"), device=DEV)
        kvc.kvc_decode_attn(cache, q, q_slot, out, lse, ws)
        torch.cuda.synchronize()
        ro, rl = oracle_decode(cache, q, q_slot)
        assert np.abs(to_np(out) - ro).max() <= 2e-2
        assert np.abs(to_np(lse) - rl).max() <= 1e-3
        assert int(ws[:4 * kvc.ATTN_COUNTERS].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: f"nb{c[0]}h{c[1]}/{c[2]}T{c[3]}q{c[4]}")
def test_decode_attn_bf16(case):
    nb, hq, hkv, T, nq, q_slot = case
    say("decode bf16", case)
    cache = make_cache(2, nb, hkv, T, seed=T)
    q = kvc_synth.queries((nq, nb, hq, 128), device=DEV, seed=T + 1)
    out, lse = run_decode(cache, q, q_slot)
    ref, ref_lse = oracle_decode(cache, q, q_slot)
    err = np.abs(to_np(out) - ref).max()
    lerr = np.abs(to_np(lse) - ref_lse).max()
    say(f"  max|o-ref| = {err:.3e}  max|lse-ref| = {lerr:.3e}")
    assert err <= 2e-2
    assert err <= 1e-3          # the hi/lo split of P keeps it near fp32 level
    assert lerr <= 1e-4


@pytest.mark.parametrize("T", [1, 64, 1024, 1031])
def test_decode_attn_f32_tiny(T):
    say("decode f32", T)
    cache = make_cache(1, 1, 2, T, dtype=torch.float32, seed=7)
    q = kvc_synth.queries((1, 1, 8, 128), dtype=torch.float32, device=DEV, seed=8)
    out, lse = run_decode(cache, q, [0])
    ref, ref_lse = oracle_decode(cache, q, [0])
    err = np.abs(to_np(out) - ref).max()
    say(f"  max|o-ref| / max|ref| = {err / np.abs(ref).max():.3e}")
    assert err <= 1e-5 * np.abs(ref).max()
    assert np.abs(to_np(lse) - ref_lse).max() <= 1e-5 * max(1.0, np.abs(ref_lse).max())


@pytest.mark.parametrize("nb", [2, 16])            # 16 x 8 slabs: value-channel halves
@pytest.mark.parametrize("T0", [95, 96, 127, 200])  # appended row ends / starts / fills a tile
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_attn_append(dtype, T0, nb):
    say("decode append", dtype, T0, nb)
    hkv, hq = 8 if dtype == torch.bfloat16 else 2, 32 if dtype == torch.bfloat16 else 8
    cache = make_cache(2, nb, hkv, T0, t_cap=256, dtype=dtype, seed=3)
    kn = kvc_synth.queries((nb, hkv, 128), dtype=dtype, device=DEV, seed=11)
    vn = kvc_synth.queries((nb, hkv, 128), dtype=dtype, device=DEV, seed=12) * 3
    K0, V0 = slab_np(cache, 1)
    cache.t_len = T0 + 1
    q = kvc_synth.queries((2, nb, hq, 128), dtype=dtype, device=DEV, seed=13)
    out, lse = run_decode(cache, q, [1, 1], k_new=kn, v_new=vn, append_slot=1)
    # the cache row was written
    assert torch.equal(cache.k[1, :, :, T0, :], kn)
    assert torch.equal(cache.v_row(1, T0), vn)
    K = np.concatenate([K0, to_np(kn)[:, :, None]], axis=2)
    V = np.concatenate([V0, to_np(vn)[:, :, None]], axis=2)
    ref, ref_lse = oracle.decode_attention(to_np(q), [None, K], [None, V], [1, 1], hkv, T0 + 1)
    err = np.abs(to_np(out) - ref).max()
    tol = 2e-2 if dtype == torch.bfloat16 else 1e-5 * np.abs(ref).max()
    assert err <= tol
    # append with no q-layer on that slot still writes the row
    kn2 = kvc_synth.queries((nb, hkv, 128), dtype=dtype, device=DEV, seed=14)
    cache.t_len = T0 + 2
    run_decode(cache, q[:1], [0], k_new=kn2, v_new=kn2, append_slot=1)
    assert torch.equal(cache.k[1, :, :, T0 + 1, :], kn2)
    kvc.kvc_append(cache, 0, kn2, kn2)
    torch.cuda.synchronize()
    assert torch.equal(cache.v_row(0, T0 + 1), kn2)


def test_decode_attn_strided_layers_and_determinism():
    say("decode strided")
    nb, hq, hkv, T = 2, 32, 8, 700
    cache = make_cache(1, nb, hkv, T, seed=21)
    pool = kvc_synth.queries((4, 6, nb, hq, 128), device=DEV, seed=22)   # [layer][step]...
    q = pool[:, 2]                                                      # strided view
    lse_pool = torch.full((4, 6, nb, hq), float("nan"), device=DEV)
    out = torch.empty((4, nb, hq, 128), device=DEV)
    ws = ws_tensor(kvc.kvc_decode_attn_ws_bytes(cache, 4, hq))
    kvc.kvc_decode_attn(cache, q, [0] * 4, out, lse_pool[:, 2], ws,
                        q_layer_stride=6 * nb * hq * 128, lse_layer_stride=6 * nb * hq)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_decode(cache, q.contiguous(), [0] * 4)
    assert np.abs(to_np(out) - ref).max() <= 1e-3
    assert np.abs(to_np(lse_pool[:, 2]) - ref_lse).max() <= 1e-4
    assert torch.isnan(lse_pool[:, 1]).all() and torch.isnan(lse_pool[:, 3]).all()
    out2 = torch.empty_like(out)
    kvc.kvc_decode_attn(cache, q, [0] * 4, out2, None, ws, q_layer_stride=6 * nb * hq * 128)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_philox_words_bit_exact():
    say("philox")
    n = 1 << 16
    for (c1, c2, c3, seed) in [(0, 0, 0, 0), (3, 17, 5, 12345), (7, 35, 15, 2**63 + 99)]:
        out = torch.zeros((n, 4), dtype=torch.int32, device=DEV)
        kvc.kvc_philox_words(n, c1, c2, c3, seed, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint32).astype(np.uint64)
        k0, k1 = oracle.seed_key(seed)
        ref = np.stack(oracle.philox4x32_10(np.arange(n, dtype=np.uint64), c1, c2, c3, k0, k1), 1)
        assert np.array_equal(got, ref)


@pytest.mark.parametrize("dtype,T", [(torch.bfloat16, 1), (torch.bfloat16, 777),
                                     (torch.bfloat16, 8448), (torch.float32, 1024)])
def test_value_range_bit_exact(dtype, T):
    say("range", dtype, T)
    cache = make_cache(2, 2, 4, T, dtype=dtype, seed=5)
    rng = torch.empty((2, 4, T), device=DEV)
    kvc.kvc_value_range(cache, 1, rng)
    torch.cuda.synchronize()
    _, V = slab_np(cache, 1)
    ref = oracle.value_range(V.reshape(-1, 128)).astype(np.float32).reshape(2, 4, T)
    assert np.array_equal(rng.cpu().numpy(), ref)


def gpu_window_lse(cache, slot, q_obs):
    """Log-normalisers of the window rows as the decode kernel returns them:
    row i is decoded against the first T - w + i + 1 rows."""
    w, nb, hq, _ = q_obs.shape
    T = cache.t_len
    lse = torch.empty((w, nb, hq), device=DEV)
    out = torch.empty((1, nb, hq, 128), device=DEV)
    ws = ws_tensor(kvc.kvc_decode_attn_ws_bytes(cache, 1, hq))
    for i in range(w):
        cache.t_len = T - w + i + 1
        kvc.kvc_decode_attn(cache, q_obs[i:i + 1], [slot], out, lse[i:i + 1], ws)
    cache.t_len = T
    torch.cuda.synchronize()
    return lse


SCORE_CASES = [
    # (dtype, nb, hq, hkv, T, w, use_lse)
    (torch.bfloat16, 1, 8, 2, 32, 32, False),
    (torch.bfloat16, 2, 32, 8, 1000, 32, False),
    (torch.bfloat16, 1, 40, 8, 2113, 32, False),
    (torch.bfloat16, 2, 32, 8, 1500, 32, True),
    (torch.bfloat16, 1, 16, 8, 300, 5, True),
    (torch.bfloat16, 1, 32, 8, 8448, 32, True),      # Llama-3.1-8B steady pass length
    (torch.bfloat16, 1, 40, 8, 33280, 32, True),     # Qwen3-14B steady pass: g 5, 160 rows
    (torch.bfloat16, 2, 40, 8, 777, 16, False),      # 80 rows: an odd number of 16-row blocks
    (torch.bfloat16, 1, 64, 8, 900, 40, False),      # 320 rows: the per-head statistics pass
    (torch.bfloat16, 1, 40, 8, 40000, 32, False),    # a prompt-sized slab, 160 rows
    (torch.bfloat16, 1, 10, 2, 262144, 32, False),   # 256K rows, g 5, statistics pass
    (torch.float32, 1, 8, 2, 1024, 32, False),
    (torch.float32, 1, 8, 2, 1024, 32, True),
]


@pytest.mark.parametrize("case", SCORE_CASES,
                         ids=lambda c: f"{str(c[0])[6:]}nb{c[1]}h{c[2]}/{c[3]}T{c[4]}w{c[5]}{'L' if c[6] else ''}")
def test_score_and_fused_range(case):
    dtype, nb, hq, hkv, T, w, use_lse = case
    say("score", case)
    cache = make_cache(2, nb, hkv, T, dtype=dtype, seed=T + w)
    q_obs = kvc_synth.queries((w, nb, hq, 128), dtype=dtype, device=DEV, seed=T)
    lse = gpu_window_lse(cache, 1, q_obs) if use_lse else None
    score = torch.full((nb, hkv, T), float("nan"), device=DEV)
    rng = torch.full((nb, hkv, T), float("nan"), device=DEV)
    ws = None if use_lse else ws_tensor(kvc.kvc_score_ws_bytes(cache, hq, w))
    kvc.kvc_score(cache, 1, q_obs, score, rng, lse, ws)
    torch.cuda.synchronize()
    K, V = slab_np(cache, 1)
    qn = to_np(q_obs)
    g = hq // hkv
    worst = 0.0
    for b in range(nb):
        for j in range(hkv):
            ref = oracle.window_score(qn[:, b, j * g:(j + 1) * g], K[b, j], T)
            got = score[b, j].double().cpu().numpy()
            rel = np.abs(got - ref) / np.maximum(ref, 1e-30)
            worst = max(worst, float(np.max(rel[ref > 1e-30])))
            assert got.sum() == pytest.approx(g * w, rel=1e-4)
            rref = oracle.value_range(V[b, j]).astype(np.float32)
            assert np.array_equal(rng[b, j].cpu().numpy(), rref)
    say(f"  max relative score error {worst:.3e}")
    assert worst <= 1e-5


SELECT_CASES = [
    # (nb, hkv, T, K, B, N_v)
    (1, 2, 1024, 256, 32, 16),
    (2, 8, 4352, 4096, 128, 64),
    (1, 8, 8448, 8192, 128, 128),
    (1, 2, 32768, 8192, 128, 128),
    (1, 2, 33280, 32768, 256, 256),      # Qwen3-14B steady pass
    (1, 1, 36864, 32768, 256, 256),      # the longest slab whose keys stay in LDS
    (1, 1, 36865, 32768, 256, 256),      # one row more: keys in the workspace
    (1, 2, 262144, 65536, 512, 512),     # 256K rows
    (1, 1, 300, 100, 0, 0),
    (1, 1, 300, 100, 10, 100),
    (1, 2, 200, 250, 32, 16),            # keep everything
    (1, 1, 8, 3, 0, 0),
]


@pytest.mark.parametrize("case", SELECT_CASES, ids=lambda c: "x".join(map(str, c)))
def test_select_matches_oracle(case):
    nb, hkv, T, K, B, Nv = case
    say("select", case)
    g = torch.Generator(device=DEV).manual_seed(T + K)
    score = (torch.rand((nb, hkv, T), generator=g, device=DEV) ** 3) * 2.0
    score[..., ::97] = 0.0                                  # some zero weights
    rng = torch.rand((nb, hkv, T), generator=g, device=DEV) * 10
    rng[..., 5:9] = rng[..., 5:6]                          # exact range ties
    n_keep = min(T, K + B)
    kept = torch.full((nb, hkv, n_keep), -7, dtype=torch.int32, device=DEV)
    ws = ws_tensor(kvc.kvc_select_ws_bytes(nb, hkv, T))
    seed, layer = 1234 + T, 5
    kvc.kvc_select(score, rng, nb, hkv, T, K, B, Nv, seed, layer, kept, ws)
    torch.cuda.synchronize()
    sc, rg, kp = to_np(score), rng.cpu().numpy(), kept.cpu().numpy()
    ties = 0
    for b in range(nb):
        for j in range(hkv):
            d = oracle.select_detail(sc[b, j], rg[b, j], T, K, B, Nv, seed, layer, b, j)
            assert np.all(np.diff(kp[b, j]) > 0)
            t, bad = band_compare(kp[b, j], d)
            ties += t
            assert bad == 0
    say(f"  ties within the band: {ties}")


@pytest.mark.parametrize("case", [
    # (nb, hkv, T, K, B, N_v): ranges of four values only (thousands of rows
    # tied at the N_v threshold), half of the weights zero (infinite keys:
    # the sampling threshold itself is +inf, taken in row order)
    (1, 2, 5000, 4000, 64, 256),
    (2, 1, 40000, 32768, 256, 256),      # the same in the workspace path
    (1, 1, 3000, 2000, 0, 1999),         # N_v = K - 1: one sampled row
])
def test_select_heavy_ties(case):
    nb, hkv, T, K, B, Nv = case
    say("select ties", case)
    g = torch.Generator(device=DEV).manual_seed(T)
    score = torch.rand((nb, hkv, T), generator=g, device=DEV)
    score[..., 1::2] = 0.0
    rng = torch.floor(torch.rand((nb, hkv, T), generator=g, device=DEV) * 4)
    n_keep = min(T, K + B)
    kept = torch.full((nb, hkv, n_keep), -7, dtype=torch.int32, device=DEV)
    seed, layer = 77, 9
    kvc.kvc_select(score, rng, nb, hkv, T, K, B, Nv, seed, layer, kept,
                   ws_tensor(kvc.kvc_select_ws_bytes(nb, hkv, T)))
    torch.cuda.synchronize()
    sc, rg, kp = to_np(score), rng.cpu().numpy(), kept.cpu().numpy()
    for b in range(nb):
        for j in range(hkv):
            d = oracle.select_detail(sc[b, j], rg[b, j], T, K, B, Nv, seed, layer, b, j)
            assert np.array_equal(kp[b, j], d["kept"]), (b, j)
    say("  kept sets equal")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("pattern", ["sparse", "dense", "unordered"])
def test_compact_bit_exact(dtype, pattern):
    """sparse: 600 of 1000 rows; dense: 985 of 1000 (a steady-state pass,
    the last 64-row block ragged); unordered: the dense rows shuffled within
    each slab, so rows fall outside the staged source tiles."""
    say("compact", dtype, pattern)
    nb, hkv, T = 2, 4, 1000
    src = make_cache(2, nb, hkv, T, dtype=dtype, seed=9)
    dst = kvc.Cache.empty(2, nb, hkv, 1024, dtype=dtype, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(1)
    n_keep = 600 if pattern == "sparse" else 985
    kept = torch.stack([torch.stack([torch.randperm(T, generator=g)[:n_keep].sort().values
                                     for _ in range(hkv)]) for _ in range(nb)])
    if pattern == "unordered":
        kept = kept[..., torch.randperm(n_keep, generator=g)]
    kept = kept.int().contiguous().to(DEV)
    kept[1, 2, 7] = T + 5                                   # out of range -> zero row
    kvc.kvc_compact(src, 1, kept, n_keep, dst)
    torch.cuda.synchronize()
    dst.t_len = n_keep
    K, V = slab_np(src, 1)
    Kd, Vd = slab_np(dst, 1)
    kp = kept.cpu().numpy()
    for b in range(nb):
        for j in range(hkv):
            rows = kp[b, j]
            ok = rows < T
            Kr, Vr = oracle.compact(K[b, j], V[b, j], rows[ok])
            assert np.array_equal(Kd[b, j][ok], Kr) and np.array_equal(Vd[b, j][ok], Vr)
            # an index past the slab's rows gives a zero row (library contract)
            assert np.all(Kd[b, j][~ok] == 0) and np.all(Vd[b, j][~ok] == 0)
    assert not np.all(kp[1, 2] < T)


def test_select_sampling_law_gpu():
    """10^4 draws of the 8-token, k = 3 weighted sampling through kvc_select:
    every draw equals the oracle's, and the inclusion frequencies and the
    56-subset distribution match the enumerated law."""
    import itertools
    from scipy import stats
    say("select law")
    w = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 9.0])
    W = w.sum()
    pi = np.zeros(8)
    psub = {}
    for a, b_, c in itertools.permutations(range(8), 3):
        pr = w[a] / W * w[b_] / (W - w[a]) * w[c] / (W - w[a] - w[b_])
        pi[[a, b_, c]] += pr
        key = tuple(sorted((a, b_, c)))
        psub[key] = psub.get(key, 0.0) + pr
    nbat, calls = 100, 100
    score = torch.tensor(w, dtype=torch.float32, device=DEV).repeat(nbat, 1, 1)
    rng = torch.zeros_like(score)
    kept = torch.empty((nbat, 1, 3), dtype=torch.int32, device=DEV)
    ws = ws_tensor(kvc.kvc_select_ws_bytes(nbat, 1, 8))
    freq = np.zeros(8)
    sub_counts = {k: 0 for k in psub}
    for seed in range(calls):
        kvc.kvc_select(score, rng, nbat, 1, 8, 3, 0, 0, seed, 4, kept, ws)
        torch.cuda.synchronize()
        kp = kept.cpu().numpy()
        for b in range(nbat):
            ref = oracle.select(w, np.zeros(8), 8, 3, 0, 0, seed, 4, b, 0)
            assert np.array_equal(kp[b, 0], ref), (seed, b)
            freq[kp[b, 0]] += 1
            sub_counts[tuple(kp[b, 0].tolist())] += 1
    n = nbat * calls
    sigma = np.sqrt(n * pi * (1 - pi))
    assert np.all(np.abs(freq - n * pi) <= 4 * sigma)
    obs = np.array([sub_counts[k] for k in psub])
    exp = np.array([psub[k] for k in psub]) * n
    assert stats.chi2.sf(((obs - exp) ** 2 / exp).sum(), 55) > 1e-3

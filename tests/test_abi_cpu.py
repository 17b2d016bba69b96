"""C-ABI checks that need no GPU: exports, host-only share map, validation.

Every error path exercised here returns before the library enqueues any
device work, so fake (but aligned) device addresses are safe."""
import ctypes
import itertools
import os
import re

import pytest
import torch

import oracle
import decode_attention_kvc_amd as kvc
from decode_attention_kvc_amd._lib import kvc_cache

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "kvc.h")
L = kvc.lib()
FAKE = 0x7F0000000000          # 16-byte aligned, never dereferenced
FAKE2 = 0x7F8000000000


def header_exports():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(kvc_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = header_exports()
    assert len(names) >= 13
    assert sorted(names) == sorted(kvc.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strerror():
    assert kvc.kvc_version() == 10000
    for code in range(0, -7, -1):
        assert kvc.kvc_strerror(code)
    assert kvc.kvc_strerror(-99) == "unknown status"


def test_share_map_matches_oracle_exhaustively():
    for n in range(1, 9):
        for r in range(0, n):
            for rest in itertools.combinations(range(1, n), r):
                S = [0, *rest]
                src, slot = kvc.kvc_share_map(n, S)
                osrc, oslot = oracle.share_map(n, S)
                assert src == osrc.tolist() and slot == oslot.tolist()


@pytest.mark.parametrize("bad", [[1], [0, 0], [0, 5, 3], [0, 8], [2, 4]])
def test_share_map_rejects_bad_sets(bad):
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_share_map(8, bad)
    assert e.value.status == kvc.KVC_EINVAL


def test_share_map_page_configs():
    # 9 of 36, every 4th of 32, every 2nd of 40, all 36
    for L_, S in [(36, range(0, 36, 4)), (32, range(0, 32, 4)), (40, range(0, 40, 2)),
                  (36, range(36))]:
        src, slot = kvc.kvc_share_map(L_, list(S))
        assert max(slot) + 1 == len(list(S))


def cache(**kw):
    c = dict(k=FAKE, v=FAKE2, dtype=1, n_slots=2, nb=1, n_kv_heads=2, head_dim=128,
             t_len=100, t_cap=128)
    c.update(kw)
    return kvc_cache(c["k"], c["v"], c["dtype"], c["n_slots"], c["nb"], c["n_kv_heads"],
                     c["head_dim"], c["t_len"], c["t_cap"])


def attn(c, **kw):
    a = dict(q=FAKE, qs=0, nq=1, slots=[0], hq=8, scale=0.0, kn=None, vn=None, app=-1,
             out=FAKE, os=0, lse=None, ls=0, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    arr = (ctypes.c_int32 * max(1, len(a["slots"])))(*a["slots"])
    return L.kvc_decode_attn(ctypes.byref(c), a["q"], a["qs"], a["nq"], arr, a["hq"], a["scale"],
                             a["kn"], a["vn"], a["app"], a["out"], a["os"], a["lse"], a["ls"],
                             a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), kvc.KVC_EDTYPE),
    (dict(head_dim=64), kvc.KVC_EINVAL),
    (dict(t_len=200), kvc.KVC_EINVAL),
    (dict(t_cap=100, t_len=10), kvc.KVC_EINVAL),
    (dict(k=FAKE + 8), kvc.KVC_EALIGN),
    (dict(v=0), kvc.KVC_EALIGN),
    (dict(n_slots=0), kvc.KVC_EINVAL),
    (dict(t_len=0), kvc.KVC_EINVAL),
])
def test_decode_attn_rejects_bad_cache(kw, code):
    assert attn(cache(**kw)) == code


@pytest.mark.parametrize("kw,code", [
    (dict(hq=7), kvc.KVC_EINVAL),                       # Hq % Hkv != 0
    (dict(hq=2 * 65), kvc.KVC_EINVAL),                  # group larger than 64
    (dict(slots=[2]), kvc.KVC_EINVAL),                  # q-slot out of range
    (dict(slots=[-1]), kvc.KVC_EINVAL),
    (dict(app=2), kvc.KVC_EINVAL),                      # append slot out of range
    (dict(app=0), kvc.KVC_EALIGN),                      # append without k_new/v_new
    (dict(q=FAKE + 2), kvc.KVC_EALIGN),
    (dict(out=0), kvc.KVC_EALIGN),
    (dict(qs=5), kvc.KVC_EINVAL),                       # stride below packed size
    (dict(qs=8 * 128 + 3), kvc.KVC_EALIGN),             # stride breaks 16-byte loads
    (dict(ws=0), kvc.KVC_EWORKSPACE),
    (dict(wsb=16), kvc.KVC_EWORKSPACE),
    (dict(scale=-1.0), kvc.KVC_EINVAL),
    (dict(scale=float("nan")), kvc.KVC_EINVAL),
    (dict(nq=-1), kvc.KVC_EINVAL),
])
def test_decode_attn_rejects_bad_args(kw, code):
    assert attn(cache(), **kw) == code


def test_decode_attn_empty_inputs_are_noops():
    assert attn(cache(), nq=0, slots=[]) == kvc.KVC_OK
    assert attn(cache(nb=0)) == kvc.KVC_OK


def test_ws_bytes_queries():
    c = cache(t_len=0, t_cap=4096)
    n = ctypes.c_size_t()
    assert L.kvc_decode_attn_ws_bytes(ctypes.byref(c), 4, 8, ctypes.byref(n)) == 0
    assert n.value > 0
    assert L.kvc_decode_attn_ws_bytes(ctypes.byref(c), 1, 7, ctypes.byref(n)) == kvc.KVC_EINVAL
    assert L.kvc_score_ws_bytes(ctypes.byref(c), 8, 32, ctypes.byref(n)) == 0 and n.value > 0
    assert L.kvc_select_ws_bytes(2, 8, 1000, ctypes.byref(n)) == 0 and n.value == 2 * (2 * 8 * 1000 * 4)
    assert L.kvc_select_ws_bytes(2, 0, 1000, ctypes.byref(n)) == kvc.KVC_EINVAL


def score(c, **kw):
    a = dict(slot=0, q=FAKE, hq=8, w=32, scale=0.0, lse=None, sc=FAKE, rg=None, ws=None, wsb=0)
    a.update(kw)
    return L.kvc_score(ctypes.byref(c), a["slot"], a["q"], a["hq"], a["w"], a["scale"], a["lse"],
                       a["sc"], a["rg"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(slot=2), kvc.KVC_EINVAL),
    (dict(w=101), kvc.KVC_EINVAL),                      # window longer than the cache
    (dict(w=0), kvc.KVC_EINVAL),
    (dict(hq=2 * 17, w=32), kvc.KVC_EINVAL),            # g*w > 512
    (dict(hq=9), kvc.KVC_EINVAL),
    (dict(q=FAKE + 4), kvc.KVC_EALIGN),
    (dict(sc=0), kvc.KVC_EALIGN),
    (dict(), kvc.KVC_EWORKSPACE),                       # two-pass needs a workspace
])
def test_score_rejects_bad_args(kw, code):
    assert score(cache(), **kw) == code


def test_score_f32_row_cap():
    assert score(cache(dtype=0), hq=2 * 5, w=32) == kvc.KVC_EINVAL   # 5*32 > 128 on f32


def select(**kw):
    a = dict(sc=FAKE, rg=FAKE2, nb=1, h=2, T=300, K=100, B=10, nv=5, seed=0, layer=0,
             kept=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return L.kvc_select(a["sc"], a["rg"], a["nb"], a["h"], a["T"], a["K"], a["B"], a["nv"],
                        a["seed"], a["layer"], a["kept"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(nv=101), kvc.KVC_EINVAL),
    (dict(nv=-1), kvc.KVC_EINVAL),
    (dict(B=-1), kvc.KVC_EINVAL),
    (dict(K=0, B=0, nv=0), kvc.KVC_EINVAL),
    (dict(h=0), kvc.KVC_EINVAL),
    (dict(layer=-3), kvc.KVC_EINVAL),
    (dict(wsb=100), kvc.KVC_EWORKSPACE),
    (dict(ws=None), kvc.KVC_EWORKSPACE),
    (dict(kept=FAKE + 2), kvc.KVC_EALIGN),
    (dict(rg=None), kvc.KVC_EALIGN),
])
def test_select_rejects_bad_args(kw, code):
    assert select(**kw) == code


def test_select_empty_is_noop():
    assert select(T=0) == kvc.KVC_OK
    assert select(nb=0) == kvc.KVC_OK


def compact(src, dst, **kw):
    a = dict(slot=0, kept=FAKE, n=50)
    a.update(kw)
    return L.kvc_compact(ctypes.byref(src), a["slot"], a["kept"], a["n"], ctypes.byref(dst), None)


def test_compact_validation():
    src = cache(k=0x10000000, v=0x20000000)
    dst = cache(k=0x30000000, v=0x40000000)
    assert compact(src, cache(k=0x10000000 + 64, v=0x40000000)) == kvc.KVC_EALIAS
    assert compact(src, cache(k=0x30000000, v=0x20000000)) == kvc.KVC_EALIAS
    assert compact(src, cache(k=0x30000000, v=0x30000000)) == kvc.KVC_EALIAS
    assert compact(src, cache(k=0x30000000, v=0x40000000, dtype=0)) == kvc.KVC_EDTYPE
    assert compact(src, cache(k=0x30000000, v=0x40000000, nb=2)) == kvc.KVC_EINVAL
    assert compact(src, dst, n=101) == kvc.KVC_EINVAL      # more than src t_len
    assert compact(src, cache(k=0x30000000, v=0x40000000, t_cap=64, t_len=0), n=65) == kvc.KVC_EINVAL
    assert compact(src, dst, slot=2) == kvc.KVC_EINVAL
    assert compact(src, dst, kept=FAKE + 1) == kvc.KVC_EALIGN
    assert compact(src, dst, n=0) == kvc.KVC_OK


def test_append_and_range_and_philox_validation():
    c = cache()
    assert L.kvc_append(ctypes.byref(c), 2, FAKE, FAKE, None) == kvc.KVC_EINVAL
    assert L.kvc_append(ctypes.byref(c), 0, None, FAKE, None) == kvc.KVC_EALIGN
    assert L.kvc_append(ctypes.byref(cache(t_len=0)), 0, FAKE, FAKE, None) == kvc.KVC_EINVAL
    assert L.kvc_value_range(ctypes.byref(c), -1, FAKE, None) == kvc.KVC_EINVAL
    assert L.kvc_value_range(ctypes.byref(c), 0, FAKE + 1, None) == kvc.KVC_EALIGN
    assert L.kvc_value_range(ctypes.byref(cache(t_len=0)), 0, FAKE, None) == kvc.KVC_OK
    assert L.kvc_philox_words(-1, 0, 0, 0, 0, FAKE, None) == kvc.KVC_EINVAL
    assert L.kvc_philox_words(4, 0, 0, 0, 0, FAKE + 4, None) == kvc.KVC_EALIGN
    assert L.kvc_philox_words(0, 0, 0, 0, 0, FAKE, None) == kvc.KVC_OK
    # read probe: a whole number of 16-byte words, aligned buffers
    assert L.kvc_read_probe(FAKE, 17, FAKE, None) == kvc.KVC_EINVAL
    assert L.kvc_read_probe(FAKE + 4, 32, FAKE, None) == kvc.KVC_EALIGN
    assert L.kvc_read_probe(FAKE, 32, FAKE + 1, None) == kvc.KVC_EALIGN
    assert L.kvc_read_probe(FAKE, 32, None, None) == kvc.KVC_EALIGN
    with pytest.raises(ValueError):
        kvc.kvc_read_probe(torch.zeros(16), torch.zeros(kvc.PROBE_BLOCKS, dtype=torch.int32))
    assert L.kvc_decode_attn(None, FAKE, 0, 1, (ctypes.c_int32 * 1)(0), 8, 0.0, None, None, -1,
                             FAKE, 0, None, 0, FAKE, 1 << 30, None) == kvc.KVC_EALIGN


@pytest.mark.parametrize("T", [1, 31, 32, 95, 128])
def test_cache_layout_roundtrip(T):
    import torch
    c = kvc.Cache.empty(2, 2, 3, T, dtype=torch.float32, device="cpu")
    c.v.fill_(float("nan"))
    K = torch.randn(2, 3, T, 128)
    V = torch.randn(2, 3, T, 128)
    c.fill(1, K, V)
    assert torch.equal(c.k_rows(1), K) and torch.equal(c.v_rows(1), V)
    for t in (0, T - 1):
        assert torch.equal(c.v_row(1, t), V[:, :, t])
    # element offset of V[t][d] inside a slab: (t/32)*128*32 + d*32 + t%32
    flat = c.v[1, 1, 2].reshape(-1)
    t, d = T - 1, 77
    assert flat[(t // 32) * 4096 + d * 32 + t % 32] == V[1, 2, t, d]
    if T % 32:
        assert torch.isnan(c.v[1, :, :, T // 32, :, T % 32:]).all()   # rows past T untouched


def dkv(c, **kw):
    a = dict(slot=0, g=FAKE, rank=32, sc=FAKE, rg=None, ws=FAKE2, wsb=1 << 40)
    a.update(kw)
    return L.kvc_dkv_score(ctypes.byref(c), a["slot"], a["g"], a["rank"], a["sc"], a["rg"],
                           a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(slot=2), kvc.KVC_EINVAL),
    (dict(rank=24), kvc.KVC_EINVAL),
    (dict(rank=64), kvc.KVC_EINVAL),
    (dict(g=FAKE + 4), kvc.KVC_EALIGN),
    (dict(sc=FAKE + 2), kvc.KVC_EALIGN),
    (dict(rg=FAKE + 2), kvc.KVC_EALIGN),
    (dict(ws=None), kvc.KVC_EWORKSPACE),
    (dict(wsb=16), kvc.KVC_EWORKSPACE),
    (dict(ws=FAKE2 + 8), kvc.KVC_EWORKSPACE),
])
def test_dkv_rejects_bad_args(kw, code):
    assert dkv(cache(), **kw) == code


def test_dkv_validation_and_sizes():
    assert dkv(cache(dtype=0)) == kvc.KVC_EDTYPE
    assert dkv(cache(t_len=0)) == kvc.KVC_OK
    assert dkv(cache(nb=0)) == kvc.KVC_OK
    n16, n32 = ctypes.c_size_t(), ctypes.c_size_t()
    c = cache(nb=2, n_kv_heads=4, t_len=100, t_cap=192)
    assert L.kvc_dkv_ws_bytes(ctypes.byref(c), 16, ctypes.byref(n16)) == 0
    assert L.kvc_dkv_ws_bytes(ctypes.byref(c), 32, ctypes.byref(n32)) == 0
    # at least the sketch rows of the capacity: slabs * t_cap * rank floats
    assert n16.value >= 8 * 192 * 16 * 4 and n32.value >= 8 * 192 * 32 * 4
    assert L.kvc_dkv_ws_bytes(ctypes.byref(c), 8, ctypes.byref(n16)) == kvc.KVC_EINVAL
    assert L.kvc_gaussian_bf16(-1, 0, 0, 0, FAKE, None) == kvc.KVC_EINVAL
    assert L.kvc_gaussian_bf16((1 << 32) + 1, 0, 0, 0, FAKE, None) == kvc.KVC_EINVAL
    assert L.kvc_gaussian_bf16(4, 0, 0, 0, FAKE + 2, None) == kvc.KVC_EALIGN
    assert L.kvc_gaussian_bf16(0, 0, 0, 0, FAKE, None) == kvc.KVC_OK


def ragged_cache(nb_cap=0, batch_idx=None, seq_len=None, **kw):
    c = cache(**kw)
    c.nb_cap = nb_cap
    c.batch_idx = batch_idx
    c.seq_len = seq_len
    return c


def test_ragged_cache_validation():
    rng = lambda c: L.kvc_value_range(ctypes.byref(c), 0, FAKE, None)
    # without a map, sequence b is entry b: nb <= nb_cap
    assert rng(ragged_cache(nb=3, nb_cap=2)) == kvc.KVC_EINVAL
    assert rng(ragged_cache(nb_cap=-1)) == kvc.KVC_EINVAL
    # with a map any entry count is addressable (t_len 0: validated, nothing launched)
    assert rng(ragged_cache(nb=3, nb_cap=2, batch_idx=FAKE, t_len=0)) == kvc.KVC_OK
    assert rng(ragged_cache(nb=3, nb_cap=3, seq_len=FAKE, t_len=0)) == kvc.KVC_OK
    assert rng(ragged_cache(batch_idx=FAKE + 2)) == kvc.KVC_EALIGN
    assert rng(ragged_cache(seq_len=FAKE + 1)) == kvc.KVC_EALIGN
    assert attn(ragged_cache(seq_len=FAKE + 2)) == kvc.KVC_EALIGN


def test_select_seq_validation():
    f = lambda **kw: L.kvc_select_seq(FAKE, FAKE, 1, 2, kw.get("T", 100), kw.get("sl", None),
                                      kw.get("sid", None), 50, 8, 4, 1, 0, FAKE, FAKE, 1 << 30,
                                      None)
    assert f(sl=FAKE + 2) == kvc.KVC_EALIGN
    assert f(sid=FAKE + 1) == kvc.KVC_EALIGN
    assert f(T=0, sl=FAKE) == kvc.KVC_OK


def test_q8_quantize_rejects_ragged_sources():
    from decode_attention_kvc_amd._lib import kvc_qcache
    q = kvc_qcache(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 1, 2, 128, 100, 128, 0, 64)
    for c in (ragged_cache(seq_len=FAKE), ragged_cache(batch_idx=FAKE, nb_cap=1),
              ragged_cache(nb_cap=2)):
        assert L.kvc_q8_quantize(ctypes.byref(c), 0, None, 0, ctypes.byref(q), None) == \
            kvc.KVC_EINVAL


def test_cache_seqs_view():
    import torch
    c = kvc.Cache.empty(2, 5, 2, 64, device="cpu", t_len=10)
    idx = torch.tensor([4, 1, 3], dtype=torch.int32)
    ln = torch.tensor([7, 0, 10], dtype=torch.int32)
    v = c.seqs(idx, ln)
    assert (v.nb, v.nb_cap, c.nb, v.t_len) == (3, 5, 5, 10)
    d = v.desc()
    assert (d.nb, d.nb_cap, d.batch_idx, d.seq_len) == (3, 5, idx.data_ptr(), ln.data_ptr())
    assert c.desc().batch_idx is None and c.desc().nb_cap == 5
    with pytest.raises(ValueError):
        c.seqs(idx.long())
    with pytest.raises(ValueError):
        c.seqs(idx, ln[:2])


def xkv_desc(**kw):
    from decode_attention_kvc_amd._lib import kvc_xkv
    d = dict(ak=FAKE, av=FAKE, lk=FAKE, bk=FAKE, bv=FAKE, nb=1, n_kv_heads=2, head_dim=128,
             window=4, rank=64, chunk=8, t_len=100, t_cap=128)
    d.update(kw)
    return kvc_xkv(d["ak"], d["av"], d["lk"], d["bk"], d["bv"], d["nb"], d["n_kv_heads"],
                   d["head_dim"], d["window"], d["rank"], d["chunk"], d["t_len"], d["t_cap"])


@pytest.mark.parametrize("kw,code", [
    (dict(window=5), kvc.KVC_EINVAL), (dict(window=0), kvc.KVC_EINVAL),
    (dict(rank=48), kvc.KVC_EINVAL), (dict(chunk=4), kvc.KVC_EINVAL),
    (dict(t_cap=100), kvc.KVC_EINVAL), (dict(t_len=200), kvc.KVC_EINVAL),
    (dict(head_dim=64), kvc.KVC_EINVAL), (dict(lk=FAKE + 4), kvc.KVC_EALIGN),
])
def test_xkv_store_validation(kw, code):
    n = ctypes.c_size_t()
    assert L.kvc_xkv_factor_ws_bytes(ctypes.byref(xkv_desc(**kw)), ctypes.byref(n)) == code


def test_xkv_ws_bytes_and_factor_validation():
    n = ctypes.c_size_t()
    x = xkv_desc()
    assert L.kvc_xkv_factor_ws_bytes(ctypes.byref(x), ctypes.byref(n)) == kvc.KVC_OK
    assert n.value >= 2 * 2 * 512 * 512 * 4 + 2 * 2 * 64 * 512 * 2
    f = lambda c, slot0=0, iters=12, x=x: L.kvc_xkv_factor(ctypes.byref(c), slot0, iters, 0,
                                                           ctypes.byref(x), FAKE, 1 << 40, None)
    c4 = cache(n_slots=4, n_kv_heads=2)
    assert f(c4, slot0=1) == kvc.KVC_EINVAL                      # window past the last slot
    assert f(c4, iters=0) == kvc.KVC_EINVAL
    assert f(cache(n_slots=4, dtype=0)) == kvc.KVC_EDTYPE
    assert f(c4, x=xkv_desc(t_len=99)) == kvc.KVC_EINVAL         # lengths disagree
    assert f(c4, x=xkv_desc(n_kv_heads=1)) == kvc.KVC_EINVAL
    assert f(ragged_cache(n_slots=4, seq_len=FAKE)) == kvc.KVC_EINVAL
    assert f(cache(n_slots=4, t_len=0), x=xkv_desc(t_len=0)) == kvc.KVC_OK


def test_xkv_decode_validation():
    x = xkv_desc()
    d = lambda layer=0, hq=8, nsel=64, o_in=None, lse_in=None, q=FAKE, x=x, ws=FAKE, wsb=1 << 40: \
        L.kvc_xkv_decode_attn(ctypes.byref(x), layer, q, hq, 0.0, nsel, o_in, lse_in, FAKE, None,
                              None, ws, wsb, None)
    assert d(layer=4) == kvc.KVC_EINVAL
    assert d(hq=7) == kvc.KVC_EINVAL
    assert d(hq=2 * 9) == kvc.KVC_EINVAL                         # group of 9 heads
    assert d(nsel=0) == kvc.KVC_EINVAL
    assert d(nsel=-3) == kvc.KVC_EINVAL
    assert d(o_in=FAKE) == kvc.KVC_EINVAL                        # lse_in missing
    assert d(q=FAKE + 2) == kvc.KVC_EALIGN
    assert d(x=xkv_desc(nb=0)) == kvc.KVC_OK
    # the workspace: one arrival counter per (b, j), chunk keys, q~ and the
    # splits' partials, each part 256-byte aligned; ns = min(8, ceil(256 /
    # slabs)) workgroups per (b, j)
    def ws_expect(nb, hkv, t_len, rank):
        al = lambda v: (v + 255) // 256 * 256
        slabs = nb * hkv
        ns = min(8, -(-256 // slabs))
        nch = (t_len + 7) // 8
        return (al(slabs * 4) + al(slabs * nch * 4) + al(slabs * 8 * rank * 4)
                + slabs * ns * 8 * (rank + 2) * 4)
    n = ctypes.c_size_t()
    assert L.kvc_xkv_decode_ws_bytes(ctypes.byref(x), 8, 64, ctypes.byref(n)) == kvc.KVC_OK
    assert n.value == ws_expect(1, 2, 100, 64)
    assert d(wsb=n.value - 1) == kvc.KVC_EWORKSPACE
    assert d(ws=None) == kvc.KVC_EWORKSPACE
    assert L.kvc_xkv_decode_ws_bytes(ctypes.byref(x), 7, 64, ctypes.byref(n)) == kvc.KVC_EINVAL
    assert L.kvc_xkv_decode_ws_bytes(ctypes.byref(x), 8, 0, ctypes.byref(n)) == kvc.KVC_EINVAL
    # any n_select >= 1: at most the chunk count is kept
    assert L.kvc_xkv_decode_ws_bytes(ctypes.byref(x), 8, 600, ctypes.byref(n)) == kvc.KVC_OK
    # 25000 chunks (their keys read from the workspace, not LDS); checked
    # after the arguments
    big = xkv_desc(t_len=200000, t_cap=200000)
    assert L.kvc_xkv_decode_ws_bytes(ctypes.byref(big), 8, 64, ctypes.byref(n)) == kvc.KVC_OK
    assert n.value == ws_expect(1, 2, 200000, 64)
    assert d(x=big, wsb=n.value - 1) == kvc.KVC_EWORKSPACE
    assert d(x=big, ws=None) == kvc.KVC_EWORKSPACE
    assert d(x=big, ws=FAKE + 4) == kvc.KVC_EWORKSPACE
    x16 = xkv_desc(nb=16, n_kv_heads=8, rank=32, t_len=32768, t_cap=32768)
    assert L.kvc_xkv_decode_ws_bytes(ctypes.byref(x16), 32, 256, ctypes.byref(n)) == kvc.KVC_OK
    assert n.value == ws_expect(16, 8, 32768, 32)
    assert d(x=big, ws=None, hq=7) == kvc.KVC_EINVAL


def rows_cache(**kw):
    c = cache(**kw)
    c.v_layout = kvc.KVC_V_ROWS
    return c


def test_value_layout_validation():
    """A rows-layout cache (a prefill's [t][d] values) is refused by every
    call that reads the tiled decode layout; an unknown layout by all."""
    bad = cache()
    bad.v_layout = 2
    assert attn(bad) == kvc.KVC_EINVAL
    assert L.kvc_value_range(ctypes.byref(bad), 0, FAKE, None) == kvc.KVC_EINVAL
    r = rows_cache()
    assert attn(r) == kvc.KVC_EINVAL
    out = ctypes.c_size_t()
    assert L.kvc_decode_attn_ws_bytes(ctypes.byref(r), 1, 8, ctypes.byref(out)) == kvc.KVC_EINVAL
    assert L.kvc_append(ctypes.byref(r), 0, FAKE, FAKE, None) == kvc.KVC_EINVAL
    assert L.kvc_dkv_ws_bytes(ctypes.byref(r), 32, ctypes.byref(out)) == kvc.KVC_OK
    slots = (ctypes.c_int32 * 1)(0)
    assert L.kvc_decode_attn_noalloc(ctypes.byref(r), FAKE, 0, 1, slots, 8, 0.0, None, None, -1,
                                     FAKE, 0, None, 0, None) == kvc.KVC_EINVAL
    # compaction: a rows source passes validation, a rows destination does not
    src = rows_cache(k=0x10000000, v=0x20000000)
    assert compact(src, rows_cache(k=0x30000000, v=0x40000000)) == kvc.KVC_EINVAL
    assert compact(src, cache(k=0x30000000, v=0x40000000), n=0) == kvc.KVC_OK
    assert compact(src, cache(k=0x30000000, v=0x40000000), kept=FAKE + 2) == kvc.KVC_EALIGN
    # kept = NULL (a copy of rows [0, n)) is not an alignment error
    assert compact(src, cache(k=0x30000000, v=0x40000000), kept=None, n=0) == kvc.KVC_OK
    # the score's size and argument checks still apply to rows caches
    assert L.kvc_score_ws_bytes(ctypes.byref(r), 8, 32, ctypes.byref(out)) == kvc.KVC_OK


def test_wrappers_check_device_arguments():
    """The binding checks each device argument's element type, extent and
    layout before its pointer crosses the ABI (the C side sees pointers only);
    a host tensor is refused last."""
    import torch
    c = kvc.Cache.empty(1, 2, 2, 64, device="cpu", t_len=10)
    f32 = dict(dtype=torch.float32)
    q = torch.zeros((1, 2, 8, 128), dtype=torch.bfloat16)
    out = torch.zeros((1, 2, 8, 128), **f32)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="q: dtype"):
        kvc.kvc_decode_attn(c, q.float(), [0], out, None, ws)
    with pytest.raises(ValueError, match="out: dtype"):
        kvc.kvc_decode_attn(c, q, [0], out.bfloat16(), None, ws)
    with pytest.raises(ValueError, match="out: .* elements"):
        kvc.kvc_decode_attn(c, q, [0], out[:, :1], None, ws)
    with pytest.raises(ValueError, match="q: must be contiguous"):
        kvc.kvc_decode_attn(c, q.transpose(2, 3).contiguous().transpose(2, 3), [0], out, None, ws)
    with pytest.raises(ValueError, match="lse: .* elements"):
        kvc.kvc_decode_attn(c, q, [0], out, torch.zeros((1, 2, 7), **f32), ws)
    with pytest.raises(ValueError, match="k_new: dtype"):
        kvc.kvc_decode_attn(c, q, [0], out, None, ws, k_new=torch.zeros((2, 2, 128), **f32),
                            v_new=torch.zeros((2, 2, 128), dtype=torch.bfloat16), append_slot=0)
    with pytest.raises(ValueError, match="leave the tensor's storage"):
        kvc.kvc_decode_attn(c, q[0:1], [0, 0], out, None, ws, q_layer_stride=2 * 8 * 128,
                            out_layer_stride=2 * 8 * 128)
    with pytest.raises(ValueError, match="must be a device tensor"):
        kvc.kvc_decode_attn(c, q, [0], out, None, ws)
    # score, range, selection and compaction
    sc = torch.zeros((2, 2, 10), **f32)
    with pytest.raises(ValueError, match="range: .* elements"):
        kvc.kvc_value_range(c, 0, torch.zeros((2, 2, 5), **f32))
    with pytest.raises(ValueError, match="q_obs: shape"):
        kvc.kvc_score(c, 0, torch.zeros((4, 3, 8, 128), dtype=torch.bfloat16), sc)
    with pytest.raises(ValueError, match="score: dtype"):
        kvc.kvc_score(c, 0, torch.zeros((4, 2, 8, 128), dtype=torch.bfloat16), sc.double())
    with pytest.raises(ValueError, match="lse_obs: .* elements"):
        kvc.kvc_score(c, 0, torch.zeros((4, 2, 8, 128), dtype=torch.bfloat16), sc,
                      lse_obs=torch.zeros((4, 2, 7), **f32))
    with pytest.raises(ValueError, match="kept: dtype"):
        kvc.kvc_select(sc, sc, 2, 2, 10, 4, 2, 1, 0, 0, torch.zeros((2, 2, 6), dtype=torch.int64))
    with pytest.raises(ValueError, match="kept: .* elements"):
        kvc.kvc_select(sc, sc, 2, 2, 10, 4, 2, 1, 0, 0, torch.zeros((2, 2, 5), dtype=torch.int32))
    with pytest.raises(ValueError, match="kept: .* elements"):
        kvc.kvc_compact(c, 0, torch.zeros((2, 2, 3), dtype=torch.int32), 4, c)


def test_score_seq_validation():
    c = cache(nb=3)
    q = FAKE
    sc = FAKE2
    L_ = L
    # without an index map the query batch must cover the sequences
    assert L_.kvc_score_seq(ctypes.byref(c), 0, q, 2, None, 8, 32, 0.0, FAKE, sc, None, None, 0,
                            None) == kvc.KVC_EINVAL
    assert L_.kvc_score_seq(ctypes.byref(c), 0, q, -1, FAKE, 8, 32, 0.0, FAKE, sc, None, None, 0,
                            None) == kvc.KVC_EINVAL
    assert L_.kvc_score_seq(ctypes.byref(c), 0, q, 5, FAKE + 2, 8, 32, 0.0, FAKE, sc, None, None,
                            0, None) == kvc.KVC_EALIGN

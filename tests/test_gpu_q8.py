"""GPU parity of the range-protected int8 cache (kvc_q8_quantize,
kvc_q8_append, kvc_q8_decode_attn) against oracle/quant.py, through the C
ABI.

Bars: codes, scales and protected rows bit-exact (both sides divide in
float32 and round half to even); attention max abs error <= 2e-2 against
float64 attention over the reconstructed rows (the bf16 attention bar; the
kernel's own error is that of the bf16 path plus the float32 removal of the
code offset and fp16 queries and P halves, measured <= 1.5e-4)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import quant as oq
import kvc_synth
import decode_attention_kvc_amd as kvc
from helpers import make_cache, slab_np, ws_tensor, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def protect_list(cache, slot, P):
    """The P largest value ranges per slab, via the library (range + select)."""
    nb, hkv, T = cache.nb, cache.n_kv_heads, cache.t_len
    if P == 0:
        return None
    rng = torch.empty((nb, hkv, T), device=DEV)
    kvc.kvc_value_range(cache, slot, rng)
    kept = torch.empty((nb, hkv, P), dtype=torch.int32, device=DEV)
    kvc.kvc_select(rng, rng, nb, hkv, T, P, 0, P, 0, 0, kept,
                   ws_tensor(kvc.kvc_select_ws_bytes(nb, hkv, T)))
    return kept


def quantized(nb, hkv, T, P, n_slots=2, slot=1, seed=0, t_cap=None):
    src = make_cache(n_slots, nb, hkv, T, seed=seed)
    qc = kvc.QCache.empty(n_slots, nb, hkv, t_cap or T + 64, max(P, 1))
    # poison the destination so that unwritten bytes show
    for t in (qc.kq, qc.vq):
        t.fill_(0x5A)
    qc.sk.fill_(float("nan"))
    qc.sv.fill_(float("nan"))
    prot = protect_list(src, slot, P)
    kvc.kvc_q8_quantize(src, slot, prot, P, qc)
    torch.cuda.synchronize()
    return src, qc, prot


def codes_np(qc, slot, T):
    kq = qc.kq[slot, :, :, :T].cpu().numpy().astype(np.int16) - 128
    vq = qc.vq[slot].transpose(-1, -2).reshape(qc.nb, qc.n_kv_heads, qc.t_cap, 128)[:, :, :T]
    vq = vq.cpu().numpy().astype(np.int16) - 128
    return kq, vq


QUANT_CASES = [(2, 4, 300, 3), (1, 8, 4097, 41), (1, 2, 33, 0), (1, 1, 64, 64), (1, 2, 31, 5)]


@pytest.mark.parametrize("case", QUANT_CASES, ids=lambda c: "x".join(map(str, c)))
def test_quantize_bit_exact(case):
    nb, hkv, T, P = case
    say("q8 quantize", case)
    src, qc, prot = quantized(nb, hkv, T, P)
    K, V = slab_np(src, 1)
    kq, vq = codes_np(qc, 1, T)
    sk = qc.sk[1, :, :, :T].cpu().numpy()
    sv = qc.sv[1, :, :, :T].cpu().numpy()
    for b in range(nb):
        for j in range(hkv):
            want_p = oq.protected_rows(V[b, j], P)
            if P:
                assert np.array_equal(prot[b, j].cpu().numpy(), want_p)
            mask = np.ones(T, bool)
            mask[want_p] = False
            ck, s_k = oq.quantize_rows(K[b, j])
            cv, s_v = oq.quantize_rows(V[b, j])
            assert np.array_equal(kq[b, j][mask], ck[mask].astype(np.int16))
            assert np.array_equal(vq[b, j][mask], cv[mask].astype(np.int16))
            assert np.array_equal(sk[b, j][mask], s_k[mask])
            assert np.array_equal(sv[b, j][mask], s_v[mask])
            assert np.all(sk[b, j][~mask] < 0)
            if P:
                kp = qc.kp[1, b, j, :P].double().cpu().numpy()
                vp = kvc.Cache(qc.kp, qc.vp, P).v_rows(1)[b, j].double().cpu().numpy()
                assert np.array_equal(kp, K[b, j][want_p])
                assert np.array_equal(vp, V[b, j][want_p])


ATTN_CASES = [
    # (nb, hkv, hq, T, P, q_slots)
    (1, 2, 8, 1, 0, [1]),
    (2, 8, 32, 300, 3, [1]),
    (1, 8, 32, 4097, 41, [1]),
    (1, 8, 32, 2500, 25, [1, 1, 1, 1]),        # grouped: 16 query rows
    (2, 8, 40, 777, 8, [1, 0]),                # two slots, g = 5
    (1, 2, 8, 64, 64, [1]),                    # every row protected
    (1, 2, 8, 200, 70, [1]),                   # protected rows fill whole tiles
    (1, 8, 64, 900, 9, [1] * 4),               # 32 query rows
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: f"nb{c[0]}h{c[2]}/{c[1]}T{c[3]}P{c[4]}q{len(c[5])}")
def test_q8_attention_matches_oracle(case):
    nb, hkv, hq, T, P, q_slot = case
    say("q8 attention", case)
    src = make_cache(2, nb, hkv, T, seed=T + P)
    qc = kvc.QCache.empty(2, nb, hkv, T + 64, max(P, 1))
    for s in range(2):
        kvc.kvc_q8_quantize(src, s, protect_list(src, s, P), P, qc)
    nq = len(q_slot)
    q = kvc_synth.queries((nq, nb, hq, 128), device=DEV, seed=7)
    out = torch.full((nq, nb, hq, 128), float("nan"), device=DEV)
    lse = torch.full((nq, nb, hq), float("nan"), device=DEV)
    ws = ws_tensor(kvc.kvc_q8_decode_attn_ws_bytes(qc, nq, hq))
    kvc.kvc_q8_decode_attn(qc, q, q_slot, out, lse, ws)
    torch.cuda.synchronize()
    g = hq // hkv
    worst = worst_l = 0.0
    for i, s in enumerate(q_slot):
        K, V = slab_np(src, s)
        for b in range(nb):
            for j in range(hkv):
                qq = q[i, b, j * g:(j + 1) * g].double().cpu().numpy()
                ref, rl = oq.quantized_attention(qq, K[b, j], V[b, j], P)
                worst = max(worst, float(np.abs(to_np(out[i, b, j * g:(j + 1) * g]) - ref).max()))
                worst_l = max(worst_l, float(np.abs(to_np(lse[i, b, j * g:(j + 1) * g]) - rl).max()))
    say(f"  max|o-ref| = {worst:.3e}  max|lse-ref| = {worst_l:.3e}")
    assert worst <= 2e-2 and worst_l <= 2e-2


def test_q8_append_and_attend():
    say("q8 append")
    nb, hkv, hq, T0, P = 2, 8, 32, 95, 2
    src = make_cache(1, nb, hkv, T0, seed=3)
    qc = kvc.QCache.empty(1, nb, hkv, 192, P)
    kvc.kvc_q8_quantize(src, 0, protect_list(src, 0, P), P, qc)
    kn = kvc_synth.queries((nb, hkv, 128), device=DEV, seed=11)
    vn = kvc_synth.queries((nb, hkv, 128), device=DEV, seed=12) * 3
    qc.t_len = T0 + 1
    kvc.kvc_q8_append(qc, 0, kn, vn)
    torch.cuda.synchronize()
    ck, s_k = oq.quantize_rows(to_np(kn).reshape(-1, 128))
    cv, s_v = oq.quantize_rows(to_np(vn).reshape(-1, 128))
    kq, vq = codes_np(qc, 0, T0 + 1)
    assert np.array_equal(kq[:, :, T0].reshape(-1, 128), ck.astype(np.int16))
    assert np.array_equal(vq[:, :, T0].reshape(-1, 128), cv.astype(np.int16))
    assert np.array_equal(qc.sk[0, :, :, T0].cpu().numpy().reshape(-1), s_k)
    assert np.array_equal(qc.sv[0, :, :, T0].cpu().numpy().reshape(-1), s_v)
    # attention over the appended slab
    q = kvc_synth.queries((1, nb, hq, 128), device=DEV, seed=13)
    out = torch.empty((1, nb, hq, 128), device=DEV)
    kvc.kvc_q8_decode_attn(qc, q, [0], out, None,
                           ws_tensor(kvc.kvc_q8_decode_attn_ws_bytes(qc, 1, hq)))
    torch.cuda.synchronize()
    K, V = slab_np(src, 0)
    g = hq // hkv
    worst = 0.0
    for b in range(nb):
        for j in range(hkv):
            Kx = np.concatenate([K[b, j], to_np(kn)[b, j][None]])
            Vx = np.concatenate([V[b, j], to_np(vn)[b, j][None]])
            # the appended row is never protected: protect within the old rows
            Kh, Vh, prot = oq.reconstruct(K[b, j], V[b, j], P)
            Kh = np.concatenate([Kh, oq.dequantize_rows(ck, s_k).reshape(nb, hkv, 128)[b, j][None]])
            Vh = np.concatenate([Vh, oq.dequantize_rows(cv, s_v).reshape(nb, hkv, 128)[b, j][None]])
            ref, _ = oracle.attention(q[0, b, j * g:(j + 1) * g].double().cpu().numpy(), Kh, Vh)
            worst = max(worst, float(np.abs(to_np(out[0, b, j * g:(j + 1) * g]) - ref).max()))
    say(f"  max|o-ref| = {worst:.3e}")
    assert worst <= 2e-2

"""kvc_decode_attn_noalloc: the decode-attention entry point for callers that
cannot allocate (graph capture, tight serving loops), whose split partials
live in the library's own 32 MiB device array.  It runs the same kernels with
the same launch plan as kvc_decode_attn, so its outputs must equal that
call's bit for bit; two calls in a row (the second smaller) check that the
array's leftover contents never leak into a result."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import kvc_synth
import decode_attention_kvc_amd as kvc
from decode_attention_kvc_amd._lib import kvc_cache
from helpers import make_cache, slab_np, ws_tensor, to_np

DEV = "cuda"
FAKE, FAKE2 = 0x7F0000000000, 0x7F8000000000


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def test_noalloc_rejects_calls_beyond_its_array():
    """Host-side: a call needing more than the array holds returns
    KVC_ESCRATCH before anything is enqueued (fake device pointers are never
    touched); argument errors keep their own codes."""
    L = kvc.lib()
    slots = (ctypes.c_int32 * 1)(0)
    # 4096 batch entries x 16 kv heads = 65536 slabs: ~520 MB of partials
    c = kvc_cache(FAKE, FAKE2, kvc.KVC_BF16, 1, 4096, 16, 128, 64, 64, 4096, None, None)
    need = ctypes.c_size_t()
    assert L.kvc_decode_attn_ws_bytes(ctypes.byref(c), 1, 16, ctypes.byref(need)) == 0
    assert need.value > kvc.NOALLOC_SCRATCH_BYTES
    st = L.kvc_decode_attn_noalloc(ctypes.byref(c), FAKE, 0, 1, slots, 16, 0.0, None, None, -1,
                                   FAKE2, 0, None, 0, None)
    assert st == kvc.KVC_ESCRATCH
    assert "32 MiB" in kvc.kvc_strerror(kvc.KVC_ESCRATCH)
    # a bad head count is still an argument error
    st = L.kvc_decode_attn_noalloc(ctypes.byref(c), FAKE, 0, 1, slots, 15, 0.0, None, None, -1,
                                   FAKE2, 0, None, 0, None)
    assert st == kvc.KVC_EINVAL


def _both(cache, q, q_slot, append=None):
    """Outputs of the workspace call and of the no-allocation call on the
    same inputs; with append=(k_new, v_new, slot) each call runs on its own
    copy of the cache, which is returned too."""
    nq, nb, hq = q.shape[0], q.shape[1], q.shape[2]
    res = []
    for noalloc in (False, True):
        c = cache
        if append is not None:
            c = kvc.Cache(cache.k.clone(), cache.v.clone(), cache.t_len)
        out = torch.full((nq, nb, hq, 128), float("nan"), device=DEV)
        lse = torch.full((nq, nb, hq), float("nan"), device=DEV)
        kw = {}
        if append is not None:
            kw = dict(k_new=append[0], v_new=append[1], append_slot=append[2])
        if noalloc:
            kvc.kvc_decode_attn_noalloc(c, q, q_slot, out, lse, **kw)
        else:
            ws = ws_tensor(kvc.kvc_decode_attn_ws_bytes(c, nq, hq))
            kvc.kvc_decode_attn(c, q, q_slot, out, lse, ws, **kw)
        torch.cuda.synchronize()
        res.append((out, lse, c))
    return res


# (nb, hq, hkv, T, q_slot): the first call large, each next one smaller
CASES = [
    (4, 40, 8, 9000, [1]),             # Qwen3-14B-shaped heads (g 5), 8 splits per slab
    (16, 32, 8, 2100, [0, 0, 0, 0]),   # grouped: four q-layers of one slot, 16 rows
    (2, 32, 8, 700, [1]),              # smaller: the array holds the last call's partials
]


@pytest.mark.gpu
def test_noalloc_equals_workspace_call_twice():
    for i, (nb, hq, hkv, T, q_slot) in enumerate(CASES):
        say(f"noalloc call {i}: nb {nb} hq {hq} hkv {hkv} T {T} q-layers {len(q_slot)}")
        cache = make_cache(2, nb, hkv, T, seed=40 + i)
        q = kvc_synth.queries((len(q_slot), nb, hq, 128), device=DEV, seed=50 + i)
        (o1, l1, _), (o2, l2, _) = _both(cache, q, q_slot)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        # and within the bf16 bar of the oracle on one slab
        K, V = slab_np(cache, q_slot[0])
        g = hq // hkv
        ref, _ = oracle.attention(to_np(q[0, nb - 1, :g]), K[nb - 1, 0], V[nb - 1, 0])
        err = float(np.abs(to_np(o2[0, nb - 1, :g]) - ref).max())
        say(f"  equal to the workspace call; max |o - ref| on a sampled slab {err:.2e}")
        assert err <= 2e-2


@pytest.mark.gpu
def test_noalloc_fused_append_equals_workspace_call():
    nb, hq, hkv, T = 3, 32, 8, 1500
    say("noalloc with the fused append")
    cache = make_cache(2, nb, hkv, T, seed=7)
    cache.t_len = T               # the appended row is row T - 1
    q = kvc_synth.queries((1, nb, hq, 128), device=DEV, seed=8)
    kn = kvc_synth.queries((nb, hkv, 128), device=DEV, seed=9)
    vn = kvc_synth.queries((nb, hkv, 128), device=DEV, seed=10)
    (o1, l1, c1), (o2, l2, c2) = _both(cache, q, [1], append=(kn, vn, 1))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # bitwise: rows past t_len hold NaN bit patterns
    assert torch.equal(c1.k.view(torch.int16), c2.k.view(torch.int16))
    assert torch.equal(c1.v.view(torch.int16), c2.v.view(torch.int16))
    assert torch.equal(c2.k[1, :, :, T - 1], kn)
    assert torch.equal(c2.v_row(1, T - 1), vn)

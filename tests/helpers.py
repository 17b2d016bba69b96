"""Shared plumbing for the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

import kvc_synth
import decode_attention_kvc_amd as kvc


def make_cache(n_slots, nb, hkv, T, t_cap=None, dtype=torch.bfloat16, seed=0, device="cuda",
               outlier_frac=0.01):
    """A cache with T rows of synthetic K/V in every slot (garbage beyond T)."""
    t_cap = t_cap or T + 64
    c = kvc.Cache.empty(n_slots, nb, hkv, t_cap, dtype=dtype, device=device)
    # fill the unused capacity with NaN bit patterns to catch reads past t_len
    c.k.view(torch.int16).fill_(-1)
    c.v.view(torch.int16).fill_(-1)
    for s in range(n_slots):
        K, V, _, _ = kvc_synth.kv_slot(nb, hkv, T, dtype=dtype, device=device, seed=seed * 1000 + s,
                                       outlier_frac=outlier_frac)
        c.fill(s, K, V)
    return c


def slab_np(cache, slot):
    """Logical float64 K, V of a slot: [nb][hkv][T][d] each."""
    K = cache.k_rows(slot).double().cpu().numpy()
    V = cache.v_rows(slot).double().cpu().numpy()
    return K, V


def ws_tensor(nbytes, device="cuda"):
    return torch.zeros(max(16, (nbytes + 15) // 16 * 16), dtype=torch.uint8, device=device)


def to_np(t):
    return t.detach().double().cpu().numpy()


def band_compare(gpu_kept, detail, rel=1e-6):
    """Compare a GPU kept set with the oracle's selection of one slab.

    Returns (n_ties, n_bad): rows kept by exactly one side that are (are not)
    within `rel` of the oracle's sampling cutoff (or of the range cutoff for
    protected rows)."""
    g = set(int(x) for x in gpu_kept)
    o = set(int(x) for x in detail["kept"])
    diff = g ^ o
    ties = bad = 0
    kc = detail["kappa_cut"]
    for t in diff:
        kap = detail["kappa"][t]
        if kc is not None and np.isfinite(kap) and abs(kap - kc) <= rel * kc:
            ties += 1
        else:
            bad += 1
    return ties, bad


def dkv_tolerance(ref):
    """Bound on |score_gpu - score_ref| for the VASE-DKV leverage of one slab,
    elementwise: 1e-6 of the row's own score plus 1e-7 of the slab's largest.
    The library forms Y = [K | V] G in float32 from exact bf16 products (a
    relative error of a few 2^-24 per entry over 256 terms); the Gram matrix,
    its factorisation, the inverse factor and the quadratic form are float64,
    so the score carries the sketch's rounding (measured: at most 3.4e-7 of
    the row's own score, 1.4e-7 of the slab's largest) and one float32
    rounding of the result."""
    ref = np.asarray(ref)
    return 1e-6 * ref + 1e-7 * max(float(np.max(ref)), 1e-30)

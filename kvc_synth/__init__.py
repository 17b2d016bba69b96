"""Seeded synthetic inputs for the decode-attention / eviction workloads.

Shared by the tests, the oracle checks and the benchmark.  It draws random
tensors of the workloads' shapes and value distributions and nothing else:
no step of the method is computed here.

Recipe (the pages' models and datasets are not available, so only their
shapes are kept):
  * Q, K, V and window queries are i.i.d. N(0, 1) from a torch.Generator
    seeded with `seed` on the target device;
  * value outliers: in every (batch entry, slot, KV head) round(frac * T)
    rows, chosen uniformly without replacement, are multiplied by `scale`
    (1% and x20 by default: a heavy-tailed value range);
  * optional depth correlation between consecutive leader slots:
    X_s = rho**gap * X_{s-1} + sqrt(1 - rho**(2*gap)) * eps, i.e. a
    per-layer correlation rho applied over `gap` layers;
  * ragged batches: prompt lengths uniform in [t_min, t_max] (length_mix);
  * cross-layer low-rank caches for the factorisation path: W layers sharing
    a token basis Z (T x k) with per-layer correlated mixing and optional
    isotropic noise (lowrank_layers).
All tensors are logical: K and V as [.., T, d] rows.
"""
import math

import torch


def generator(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, dtype, device, gen):
    """N(0, 1) drawn in float32, then rounded to `dtype`."""
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dtype)


def outlier_rows(nb, hkv, T, frac, gen, device):
    """Indices [nb][hkv][n] of rows to scale, n = round(frac * T)."""
    n = int(round(frac * T))
    if n == 0:
        return torch.zeros((nb, hkv, 0), dtype=torch.long, device=device)
    u = torch.rand((nb, hkv, T), generator=gen, device=device)
    return u.topk(n, dim=-1).indices


def kv_slot(nb, hkv, T, d=128, dtype=torch.bfloat16, device="cpu", seed=0,
            outlier_frac=0.01, outlier_scale=20.0, prev=None, rho=None, gap=1):
    """K, V rows [nb][hkv][T][d] for one leader slot.

    With `prev` = (K_prev, V_prev) float32 and `rho`, the new slot is
    correlated with the previous one as described in the module docstring.
    Returns (K, V, K32, V32): the rounded tensors and the float32 draws
    before rounding (for chaining correlated slots)."""
    gen = generator(seed, device)
    k = torch.randn((nb, hkv, T, d), generator=gen, device=device)
    v = torch.randn((nb, hkv, T, d), generator=gen, device=device)
    if prev is not None and rho is not None:
        a = rho ** gap
        b = math.sqrt(1.0 - a * a)
        k = a * prev[0] + b * k
        v = a * prev[1] + b * v
    idx = outlier_rows(nb, hkv, T, outlier_frac, gen, device)
    v_out = v.clone()
    if idx.shape[-1]:
        sel = idx.unsqueeze(-1).expand(-1, -1, -1, d)
        v_out.scatter_(2, sel, v.gather(2, sel) * outlier_scale)
    return k.to(dtype), v_out.to(dtype), k, v


def append_rows(n_steps, n_slots, nb, hkv, d=128, dtype=torch.bfloat16, device="cpu", seed=0,
                outlier_frac=0.01, outlier_scale=20.0):
    """New K and V rows [n_steps][n_slots][nb][hkv][d] for a decode whose
    cache grows from empty: N(0, 1), and for every (slot, batch entry, KV
    head) round(outlier_frac * n_steps) uniformly chosen steps whose value
    row is scaled by outlier_scale (the value outliers of a prompt cache,
    spread over the generated rows).  Returns (k_new, v_new)."""
    gen = generator(seed, device)
    k = normal((n_steps, n_slots, nb, hkv, d), dtype, device, gen)
    v = torch.randn((n_steps, n_slots, nb, hkv, d), generator=gen, device=device)
    idx = outlier_rows(n_slots * nb, hkv, n_steps, outlier_frac, gen, device)
    if idx.shape[-1]:
        hit = torch.zeros((n_slots * nb, hkv, n_steps), dtype=torch.bool, device=device)
        hit.scatter_(-1, idx, True)
        hit = hit.reshape(n_slots, nb, hkv, n_steps).permute(3, 0, 1, 2)
        v[hit] *= outlier_scale
    return k, v.to(dtype)


def lowrank_layers(nb, hkv, T, W, k, noise=0.0, rho=0.9, d=128, dtype=torch.bfloat16,
                   device="cpu", seed=0):
    """K and V rows [nb][hkv][T][d] of W consecutive layers whose caches share
    a token basis: per (batch entry, KV head) and for keys and values
    separately, X_l = Z M_l + noise * E_l with Z ~ N(0, 1) of shape T x k
    shared by the layers, M_1 ~ N(0, 1/k) (k x d) and
    M_l = rho M_{l-1} + sqrt(1 - rho^2) N(0, 1/k) (a per-layer correlation),
    E_l ~ N(0, 1).  Returns a list of W (K, V) pairs."""
    gen = generator(seed, device)
    out = [[None, None] for _ in range(W)]
    for kv in range(2):
        Z = torch.randn((nb, hkv, T, k), generator=gen, device=device)
        M = torch.randn((nb, hkv, k, d), generator=gen, device=device) / math.sqrt(k)
        for l in range(W):
            if l:
                M = rho * M + math.sqrt(1 - rho * rho) * torch.randn(
                    (nb, hkv, k, d), generator=gen, device=device) / math.sqrt(k)
            X = Z @ M
            if noise:
                X = X + noise * torch.randn((nb, hkv, T, d), generator=gen, device=device)
            out[l][kv] = X.to(dtype)
    return [tuple(x) for x in out]


def length_mix(n, t_min, t_max, seed=0):
    """Prompt lengths of a ragged batch: n integers uniform in [t_min, t_max]
    (a seeded CPU generator), as a list."""
    g = generator(seed, "cpu")
    return [int(x) for x in torch.randint(t_min, t_max + 1, (n,), generator=g)]


def queries(shape, dtype=torch.bfloat16, device="cpu", seed=0):
    """Decode or window queries of any shape, N(0, 1)."""
    return normal(shape, dtype, device, generator(seed, device))

"""Decode throughput of attention + eviction over a compressed KV cache, 1 GPU.

Workload (default): Qwen3-14B-shaped long-context decode -- 40 layers, one KV
leader every 2nd layer (20 slots), batch 4, 40 query / 8 KV heads, head dim
128, bfloat16, a 128K-token prompt cache compressed once to K + B = 33024
rows, then decode steps with a VASE eviction pass (K 32768, B 256, N_v 256,
window 32, every 256 steps) on the leaders.  A step = every layer's attention
(with the leaders' fused append) + its share of the periodic eviction: the
timed steps run at the steady state's mean cache length (untimed pre-roll
steps get there), one pass at its steady-state length (K + B + period rows)
is timed with HIP events, and its time counts once per period.  Inputs are
synthetic (seeded normal draws with 1% x20 value outliers) and resident in
HBM before timing starts.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--mode ...]

Prints one JSON line.  Only the cpu_baseline leg touches oracle/.
"""
import argparse
import gc
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "decode tokens/s and achieved HBM GB/s (% of peak), attn+eviction, 1 GPU"

WORKLOADS = {
    "llama3.1-8b-combined": dict(
        desc="Llama-3.1-8B-shaped combined R-CLA sharing + VASE eviction decode",
        n_layers=32, leaders=list(range(0, 32, 4)), nb=16, hq=32, hkv=8, t0=32768,
        evict=dict(K=8192, B=128, N_v=128, w=32, period=128, seed=0)),
    "qwen3-8b-rcla": dict(
        desc="Qwen3-8B-shaped R-CLA decode, 9 of 36 layers lead, no eviction",
        n_layers=36, leaders=list(range(0, 36, 4)), nb=1, hq=32, hkv=8, t0=32768, evict=None,
        # a 135 MB slot fits the 256 MB Infinity Cache: no call follows one
        # that read the same slot
        mode="per-layer-interleaved"),
    "qwen3-4b-vase": dict(
        desc="Qwen3-4B-shaped VASE decode: every layer its own cache, 16K tokens generated "
             "from an empty cache",
        n_layers=36, leaders=list(range(36)), nb=8, hq=32, hkv=8, t0=0, steps=16384,
        evict=dict(K=4096, B=128, N_v=64, w=32, period=128, seed=0)),
    "qwen3-14b-long": dict(
        desc="Qwen3-14B-shaped long-context decode: sharing every 2 layers, 128K prompt, VASE",
        n_layers=40, leaders=list(range(0, 40, 2)), nb=4, hq=40, hkv=8, t0=131072,
        evict=dict(K=32768, B=256, N_v=256, w=32, period=256, seed=0)),
}


# The largest configuration that fits one GPU: the metric's workload.
DEFAULT_WORKLOAD = "qwen3-14b-long"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_bytes(nb, hq, hkv, t_len, n_q_layers, lead):
    """Algorithmic HBM bytes of one attention launch (bf16 cache): every K and
    V row of the slab once, queries in, float32 outputs and lse out, and the
    appended row written by leaders."""
    kv = 2 * nb * hkv * t_len * 128 * 2
    q = n_q_layers * nb * hq * 128 * 2
    out = n_q_layers * nb * hq * (128 + 1) * 4
    app = 2 * nb * hkv * 128 * 2 if lead else 0
    return kv + q + out + app


def step_attn_bytes(dec, mode, nb, hq, hkv, t_len):
    """Algorithmic bytes of one step's attention calls."""
    if mode != "grouped":
        return sum(attn_bytes(nb, hq, hkv, t_len, 1, dec.src_layer[l] == l)
                   for l in range(dec.n_layers))
    return sum(attn_bytes(nb, hq, hkv, t_len, len(g), True) for g in dec.groups)


def evict_bytes(cfg, t_len):
    """Algorithmic bytes of one eviction pass: K + V read once by the fused
    score/range pass, score/range written and read, kept rows gathered (read)
    and written; VASE-DKV adds its float32 sketch rows (written once, read
    once)."""
    e = cfg["evict"]
    slabs = cfg["nb"] * cfg["hkv"] * len(cfg["leaders"])
    keep = e["K"] + e["B"]
    sketch = 2 * 4 * e.get("rank", 32) * t_len if e.get("scoring") == "dkv" else 0
    return slabs * (2 * t_len * 256 + 2 * 4 * t_len * 2 + 4 * keep + 2 * 2 * keep * 256 + sketch)


def cpu_baseline(cfg, cache, qpool, s, budget_s=8.0):
    """Time the float64 oracle on a bounded sample of the same workload, and
    compare the library's outputs with the oracle's on that sample (the
    slabs of cache slot 0 at the bench's final cache state): decode attention
    of layer 0's queries of step s, and, for window-score eviction, the
    window scores and kept sets of one pass with the last w queries.
    Returns (baseline, parity)."""
    import numpy as np
    import torch
    import oracle
    import decode_attention_kvc_amd as kvc
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        blas = 1
    nb, hq, hkv = cfg["nb"], cfg["hq"], cfg["hkv"]
    g = hq // hkv
    T = cache.t_len
    e = cfg["evict"]
    dev = cache.k.device
    # The library's outputs on the same inputs, before any timing: layer 0's
    # decode attention (no append, the cache is unchanged) and one eviction
    # pass's window scores, ranges and kept sets on slot 0.
    g_out = torch.empty((1, nb, hq, 128), device=dev)
    kvc.kvc_decode_attn(cache, qpool[0, s:s + 1], [0], g_out, None,
                        torch.zeros(kvc.kvc_decode_attn_ws_bytes(cache, 1, hq),
                                    dtype=torch.uint8, device=dev))
    g_kept = g_score = None
    window = bool(e) and e.get("scoring", "attnv") == "attnv"
    if window:
        w = e["w"]
        g_score = torch.empty((nb, hkv, T), device=dev)
        g_rng = torch.empty((nb, hkv, T), device=dev)
        lo, hi = window_rows(s, w, qpool.shape[1])
        kvc.kvc_score(cache, 0, qpool[0, lo:hi], g_score, g_rng, None,
                      torch.zeros(kvc.kvc_score_ws_bytes(cache, hq, w), dtype=torch.uint8,
                                  device=dev))
        g_kept = torch.empty((nb, hkv, min(T, e["K"] + e["B"])), dtype=torch.int32, device=dev)
        kvc.kvc_select(g_score, g_rng, nb, hkv, T, e["K"], e["B"], e["N_v"], 1, 0, g_kept,
                       torch.empty(kvc.kvc_select_ws_bytes(nb, hkv, T), dtype=torch.uint8,
                                   device=dev))
        g_kept, g_score = g_kept.cpu().numpy(), g_score.cpu().numpy()
    g_out = g_out.cpu().numpy()
    ref_out, ref_ev = [], []
    # decode: slabs of layer 0 (slot 0), converted bf16 -> float64 per slab
    Kc = cache.k_rows(0).cpu()
    Vc = cache.v_rows(0).cpu()
    qh = qpool[0, s].cpu()
    t0 = time.perf_counter()
    n_dec = 0
    while time.perf_counter() - t0 < budget_s and n_dec < nb * hkv:
        b, j = divmod(n_dec, hkv)
        K = Kc[b, j].double().numpy()
        V = Vc[b, j].double().numpy()
        ref_out.append(oracle.attention(qh[b, j * g:(j + 1) * g].double().numpy(), K, V)[0])
        n_dec += 1
    t_dec = (time.perf_counter() - t0) / n_dec
    t_step = t_dec * cfg["n_layers"] * nb * hkv
    t_ev_total = 0.0
    n_ev = 0
    if e:
        w = e["w"]
        lo, hi = window_rows(s, w, qpool.shape[1])
        qo = qpool[0, lo:hi].cpu()
        dkv = e.get("scoring") == "dkv"
        if dkv:
            r = e.get("rank", 32)
            G = oracle.dkv.bf16_bits_to_f64(oracle.dkv.gaussian_bf16(r * 256, 1, 0, 0xFFFFFFFF))
            G = G.reshape(r, 256).T
        t1 = time.perf_counter()
        while time.perf_counter() - t1 < budget_s and n_ev < nb * hkv:
            b, j = divmod(n_ev, hkv)
            K = Kc[b, j].double().numpy()
            V = Vc[b, j].double().numpy()
            if dkv:
                sc = oracle.dkv.dkv_score(K, V, G)
            else:
                sc = oracle.window_score(qo[:, b, j * g:(j + 1) * g].double().numpy(), K, T)
            vr = oracle.value_range(V)
            det = oracle.select_detail(sc, vr, T, e["K"], e["B"], e["N_v"], 1, 0, b, j)
            oracle.compact(K, V, det["kept"])
            if not dkv:
                ref_ev.append((sc, det))
            n_ev += 1
        t_ev = (time.perf_counter() - t1) / n_ev
        t_ev_total = t_ev * nb * hkv * len(cfg["leaders"])
    per_step = t_step + (t_ev_total / e["period"] if e else 0.0)
    sample = (f"{n_dec} of {nb * hkv} slabs of one layer's decode attention at T={T}"
              + (f" and {n_ev} slabs of one eviction pass ("
                 + ("VASE-DKV leverage" if e and e.get("scoring") == "dkv" else "window score")
                 + "+range+select+compact)" if e else "")
              + f", extrapolated linearly to a full step of {cfg['n_layers']} layers"
              + (f" plus 1/{e['period']} of a pass over {len(cfg['leaders'])} leader slots"
                 if e else "")
              + "; numpy float64, bf16 converted per slab")
    baseline = dict(value=round(nb / per_step, 4), unit="tokens/s", cores=int(blas),
                    kind="oracle", sample=sample, extrapolated=True,
                    cpu_model=_cpu_model(), host_cores=len(os.sched_getaffinity(0)))

    # Parity on the sampled slabs.  Attention: max |o - o_ref| against the
    # bf16 tolerance 2e-2.  Kept sets: rows kept by one side only are ties
    # when their key lies within 1e-6 (relative) of the oracle's sampling
    # cutoff, otherwise mismatches.
    err = 0.0
    for i, ref in enumerate(ref_out):
        b, j = divmod(i, hkv)
        err = max(err, float(np.abs(g_out[0, b, j * g:(j + 1) * g] - ref).max()))
    parity = dict(sample=f"slot 0 at {T} rows, layer 0's queries of the last step",
                  attention_slabs=len(ref_out), attention_max_abs_err=float(f"{err:.3e}"),
                  attention_tol=2e-2, attention_ok=err <= 2e-2)
    if window and ref_ev:
        ties = bad = 0
        srel = 0.0
        for i, (sc, det) in enumerate(ref_ev):
            b, j = divmod(i, hkv)
            srel = max(srel, float(np.max(np.abs(g_score[b, j] - sc) / np.maximum(sc, 1e-30))))
            diff = set(g_kept[b, j].tolist()) ^ set(det["kept"].tolist())
            kc = det["kappa_cut"]
            for t in diff:
                kap = det["kappa"][t]
                if kc is not None and np.isfinite(kap) and abs(kap - kc) <= 1e-6 * kc:
                    ties += 1
                else:
                    bad += 1
        parity.update(eviction_slabs=len(ref_ev), score_max_rel_err=float(f"{srel:.3e}"),
                      kept_rows_per_slab=int(g_kept.shape[-1]), kept_ties_within_1e_6=ties,
                      kept_mismatches=bad, kept_ok=bad == 0)
    return baseline, parity


TRAFFIC_FILES = {
    "llama3.1-8b-combined": "attn_traffic_llama31_8b_combined.json",
    "qwen3-14b-long": "attn_traffic_qwen3_14b_long.json",
}


ATTN_SOURCES = ("attn.hip", "merge.h")


def attn_source_sha256():
    """sha256 of the decode attention kernel's sources (in order), the key
    under which its memory counters are recorded."""
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        h.update(open(os.path.join(ROOT, "decode_attention_kvc_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def load_traffic(workload, mode, bytes_per_launch):
    """HBM traffic per attention call from the committed counter summary of
    the same workload and call order, or None when there is none or the
    attention source has changed since the counters were taken."""
    name = TRAFFIC_FILES.get(workload)
    if name is None:
        return None, None
    path = os.path.join(ROOT, "profiles", name)
    try:
        t = json.load(open(path))
        sha = attn_source_sha256()
    except (OSError, ValueError):
        return None, None
    if t.get("attn_source_sha256") != sha or t.get("mode", "per-layer") != mode:
        return None, None
    return round(t["traffic_over_algorithmic"] * bytes_per_launch), t


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def int8_leg(args, cfg, dec, qpool, lsepool, knew, vnew, out, steps):
    """Decode attention over the range-protected int8 form of the current
    cache: the same per-layer calls (leaders append quantized rows) with no
    eviction, timed like the main leg."""
    import torch
    import decode_attention_kvc_amd as kvc
    dev = "cuda"
    c = dec.cache
    nb, hkv, hq, L = c.nb, c.n_kv_heads, cfg["hq"], cfg["n_layers"]
    n_slots = c.n_slots
    T0 = c.t_len
    P = int(math.ceil(args.protect_frac * T0))
    qc = kvc.QCache.empty(n_slots, nb, hkv, T0 + steps + 64, max(P, 1), device=dev)
    for slot in range(n_slots):
        prot = None
        if P:
            rng = torch.empty((nb, hkv, T0), device=dev)
            kvc.kvc_value_range(c, slot, rng)
            prot = torch.empty((nb, hkv, P), dtype=torch.int32, device=dev)
            kvc.kvc_select(rng, rng, nb, hkv, T0, P, 0, P, 0, 0, prot,
                           torch.empty(kvc.kvc_select_ws_bytes(nb, hkv, T0), dtype=torch.uint8,
                                       device=dev))
        kvc.kvc_q8_quantize(c, slot, prot, P, qc)
    ws = torch.zeros(max(16, kvc.kvc_q8_decode_attn_ws_bytes(qc, 1, hq)), dtype=torch.uint8,
                     device=dev)
    n_pool = qpool.shape[1]
    slots = [[x] for x in range(n_slots)]

    def step(s, events):
        qc.t_len += 1
        sp = s % n_pool
        a = b = None
        if events is not None:
            a = torch.cuda.Event(enable_timing=True)
            a.record()
        qs, ls, outs = qpool[:, sp].unbind(0), lsepool[:, sp].unbind(0), out.unbind(0)
        kn, vn = knew[sp].unbind(0), vnew[sp].unbind(0)
        for l in range(L):
            slot = dec.src_slot[l]
            if dec.src_layer[l] == l:
                kvc.kvc_q8_append(qc, slot, kn[slot], vn[slot])
            kvc.kvc_q8_decode_attn(qc, qs[l], slots[slot], outs[l], ls[l], ws, n_q_heads=hq)
        if events is not None:
            b = torch.cuda.Event(enable_timing=True)
            b.record()
            events.append((a, b, qc.t_len))

    for s in range(3):
        step(s, None)
    torch.cuda.synchronize()
    events = []
    t0 = time.perf_counter()
    for s in range(steps):
        step(3 + s, events)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sum(a.elapsed_time(b) for a, b, _ in events)
    row = 2 * (128 + 4)
    byts = sum(L * nb * hkv * (t * row + P * 2 * 256) + L * nb * hq * (128 * 2 + 129 * 4)
               for _, _, t in events)
    gbps = byts / (ms * 1e-3) / 1e9
    return dict(value=round(nb * steps / wall, 2), unit="tokens/s",
                ms_per_step=round(1e3 * wall / steps, 4),
                attention_GBps=round(gbps, 1), attention_frac=round(gbps / HBM_PEAK_GBPS, 4),
                avg_launch_us=round(1e3 * ms / (steps * L), 2), protected_rows=P,
                rows=[T0 + 4, T0 + 3 + steps], bytes_per_row=row,
                kernel="attn_q8_kernel (+ merge) and q8_append_kernel, per-layer calls, no eviction")


def ragged_leg(args, cfg, qpool, lsepool, knew, vnew, out, steps, warm=3):
    """The same model shape as a ragged batch: prompt lengths from a seeded
    length mix (uniform in [t0/16, t0]), and every sequence evicting on its own
    steps (phase b * period / nb), through RaggedDecoder.  Timed like the main
    leg; attention bytes count each sequence's own rows.  The warm-up covers
    at least one period, so that the timed steps start with every code path
    (including the first per-sequence pass) already loaded."""
    import torch
    import kvc_synth
    import decode_attention_kvc_amd as kvc
    from decode_attention_kvc_amd.loop import RaggedDecoder, ragged_plan
    dev = "cuda"
    e0 = cfg["evict"]
    L, leaders, nb, hq, hkv, tmax = (cfg[k] for k in ("n_layers", "leaders", "nb", "hq", "hkv",
                                                       "t0"))
    n_slots = len(leaders)
    warm = max(warm, e0["period"])
    if warm + steps > qpool.shape[1]:
        raise ValueError("the query pool is shorter than the ragged leg's warm-up and steps")
    t0 = kvc_synth.length_mix(nb, tmax // 16, tmax, seed=11)
    ev = dict(K=e0["K"], B=e0["B"], N_v=e0["N_v"], w=e0["w"], period=e0["period"],
              seed=e0["seed"], phase=[b * e0["period"] // nb for b in range(nb)])
    n_total = warm + steps
    mode = args.mode if args.mode in ("per-layer", "grouped") else "per-layer"
    plan = ragged_plan(t0, n_total, ev)
    prompt = kvc.Cache.empty(n_slots, nb, hkv, max(t0), device=dev, v_layout="rows")
    for s_ in range(n_slots):
        Kr, Vr, _, _ = kvc_synth.kv_slot(nb, hkv, max(t0), device=dev, seed=300 + s_)
        prompt.fill(s_, Kr, Vr)
        del Kr, Vr
    cache = kvc.Cache.empty(n_slots, plan["entries"], hkv, plan["peak"], device=dev)
    dec = RaggedDecoder(L, leaders, cache, hq, t0, n_total, ev, mode=mode)
    q_init = [kvc_synth.queries((ev["w"], nb, hq, 128), device=dev, seed=350 + i)
              for i in range(n_slots)]
    dec.initial_pass(prompt, q_init)
    torch.cuda.synchronize()
    del prompt, q_init
    for s in range(warm):
        dec.step(s, qpool, lsepool, knew, vnew, out)
    torch.cuda.synchronize()
    dec.events, dec.pass_events = [], []
    host = {True: [], False: []}         # host time of step() calls, with / without a pass
    t_start = time.perf_counter()
    for s in range(warm, n_total):
        h0 = time.perf_counter()
        dec.step(s, qpool, lsepool, knew, vnew, out)
        host[s in plan["passes"]].append(time.perf_counter() - h0)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    att_ms = sum(a.elapsed_time(b) for a, b, _, _ in dec.events)
    n_calls = sum(n for _, _, _, n in dec.events)
    rows = [sum(plan["att_len"][s]) for _, _, s, _ in dec.events]   # rows of all sequences
    per_row = 2 * hkv * 128 * 2                                         # K + V of one row, all heads
    q_out = nb * hq * (128 * 2 + 129 * 4)
    if mode == "per-layer":
        byts = sum(L * r * per_row + L * q_out + n_slots * 2 * nb * hkv * 256 for r in rows)
    else:
        byts = sum(n_slots * r * per_row + L * q_out + n_slots * 2 * nb * hkv * 256 for r in rows)
    gbps = byts / (att_ms * 1e-3) / 1e9
    pass_ms = [a.elapsed_time(b) for a, b, _, _ in dec.pass_events]
    seq_passes = sum(n for _, _, _, n in dec.pass_events)
    lens = [plan["att_len"][s] for s in range(warm, n_total)]
    return dict(value=round(nb * steps / wall, 2), unit="tokens/s",
                ms_per_step=round(1e3 * wall / steps, 4), mode=mode, warmup_steps=warm,
                attention_GBps=round(gbps, 1), attention_frac=round(gbps / HBM_PEAK_GBPS, 4),
                avg_launch_us=round(1e3 * att_ms / n_calls, 2),
                prompt_tokens=t0, phases=ev["phase"],
                rows_min_mean_max=[min(map(min, lens)), round(sum(map(sum, lens)) /
                                   (len(lens) * nb), 1), max(map(max, lens))],
                batch_entries=plan["entries"],
                eviction_passes=len(pass_ms), sequence_passes=seq_passes,
                pass_ms_mean=round(sum(pass_ms) / max(1, len(pass_ms)), 3),
                host_ms_step=round(1e3 * sum(host[False]) / max(1, len(host[False])), 3),
                host_ms_pass_step=round(1e3 * sum(host[True]) / max(1, len(host[True])), 3),
                kernel="attn_bf16_kernel (+ merge) over per-sequence lengths; passes: "
                       "score, select, compact on the due sequences only")


def xkv_leg(args, cfg, qpool, knew, vnew, steps, warm=3):
    """Cross-layer factorisation + selective reconstruction on the same model
    shape, every layer its own cache (no sharing): the 32K-row caches of each
    window of 4 layers are factorised once (rank 64, keys and values), then
    each decode step runs, per layer, attention over the rows appended since
    (kvc_decode_attn with the append, an uncompressed tail) and the selective
    reconstruction of 256 chunks of 8 rows merged into it.  Synthetic caches
    with the structure the factorisation relies on: per window, keys and
    values share a rank-48 token basis across the layers (per-layer mixing
    correlated 0.9) plus N(0, 0.1^2) noise.  Also times full attention over
    one uncompressed layer for comparison."""
    import torch
    import kvc_synth
    import decode_attention_kvc_amd as kvc
    dev = "cuda"
    L, nb, hq, hkv, T = (cfg[k] for k in ("n_layers", "nb", "hq", "hkv", "t0"))
    W, rank, n_sel, iters = 4, 64, 256, 12
    n_win = L // W
    n_slots_pool = knew.shape[1]
    stores, fact_ms = [], []
    base = None
    g = hq // hkv
    for w in range(n_win):
        layers = kvc_synth.lowrank_layers(nb, hkv, T, W, 48, noise=0.1, device=dev, seed=400 + w)
        c = kvc.Cache.empty(W, nb, hkv, T, device=dev)
        for l, (K, V) in enumerate(layers):
            c.fill(l, K, V)
        del layers, K, V
        st = kvc.XkvStore.empty(nb, hkv, W, rank, T, device=dev)
        ws = torch.empty(kvc.kvc_xkv_factor_ws_bytes(st), dtype=torch.uint8, device=dev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        kvc.kvc_xkv_factor(c, 0, st, ws, iters=iters, seed=w)
        b.record()
        torch.cuda.synchronize()
        fact_ms.append(a.elapsed_time(b))
        if w == 0:
            # full attention over one uncompressed layer of the same cache
            out1 = torch.empty((1, nb, hq, 128), device=dev)
            wsa = torch.zeros(kvc.kvc_decode_attn_ws_bytes(c, 1, hq), dtype=torch.uint8, device=dev)
            for _ in range(3):
                kvc.kvc_decode_attn(c, qpool[0, 0:1], [0], out1, None, wsa)
            torch.cuda.synchronize()
            a.record()
            for r in range(20):
                kvc.kvc_decode_attn(c, qpool[r % W, 0:1], [r % W], out1, None, wsa)
            b.record()
            torch.cuda.synchronize()
            base = a.elapsed_time(b) / 20
            del wsa, out1
        del c, ws
        stores.append(st)
    tail = kvc.Cache.empty(L, nb, hkv, warm + steps + 64, device=dev)
    tail.t_len = 0
    ws_t = torch.zeros(kvc.kvc_decode_attn_ws_bytes(tail, 1, hq), dtype=torch.uint8, device=dev)
    o_t = torch.empty((L, nb, hq, 128), device=dev)
    l_t = torch.empty((L, nb, hq), device=dev)
    out = torch.empty((L, nb, hq, 128), device=dev)
    # zeroed: the decode's arrival counters start at zero
    ws_x = torch.zeros(kvc.kvc_xkv_decode_ws_bytes(stores[0], hq, n_sel), dtype=torch.uint8,
                       device=dev)

    def step(s):
        tail.t_len += 1
        for l in range(L):
            sl = l % n_slots_pool
            kvc.kvc_decode_attn(tail, qpool[l, s], [l], o_t[l], l_t[l], ws_t, k_new=knew[s, sl],
                                v_new=vnew[s, sl], append_slot=l, n_q_heads=hq)
            kvc.kvc_xkv_decode_attn(stores[l // W], l % W, qpool[l, s], out[l], None,
                                    n_select=n_sel, o_in=o_t[l], lse_in=l_t[l], ws=ws_x)

    for s in range(warm):
        step(s)
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for s in range(warm, warm + steps):
        a = torch.cuda.Event(enable_timing=True)
        a.record()
        step(s)
        b = torch.cuda.Event(enable_timing=True)
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    nch = (T + 7) // 8
    sr_bytes = nb * hkv * (nch * rank * 2 + 2 * n_sel * 8 * rank * 2 + 2 * 128 * rank * 4
                           + g * (128 * 2 + 129 * 4 + 128 * 4))
    stored = stores[0].nbytes() * n_win
    full = 2 * L * nb * hkv * T * 128 * 2
    return dict(value=round(nb * steps / wall, 2), unit="tokens/s",
                ms_per_step=round(1e3 * wall / steps, 4), gpu_ms_per_step=round(gpu_ms, 4),
                window=W, rank=rank, chunk=8, n_select=n_sel, iters=iters, prompt_tokens=T,
                tail_rows=[warm + 1, warm + steps],
                factor_ms_per_window=round(sum(fact_ms) / len(fact_ms), 3),
                store_GB=round(stored / 1e9, 3), full_cache_GB=round(full / 1e9, 3),
                compression=round(full / stored, 2),
                sr_bytes_per_call=sr_bytes,
                full_attention_us_per_layer=round(1e3 * base, 2),
                full_attention_ms_per_step=round(L * base, 3),
                kernel="per layer: attn_bf16_kernel over the tail (+ merge), then xkv_scores + xkv_rows (two workgroups per (b, j))",
                data="synthetic cross-layer low-rank caches (rank-48 shared basis + 0.1 noise)")


def window_rows(s, w, n_pool):
    """Rows [lo, lo + w) of a query pool that form the observation window of
    a pass after step s: the w rows ending at row s, or the pool's first w
    rows while fewer than w steps have run (a slice never starts below 0)."""
    if w < 1 or n_pool < w:
        raise ValueError(f"a window of {w} rows needs a query pool of at least {w} rows "
                         f"(it has {n_pool})")
    hi = min(max(s, 0) + 1, n_pool)
    lo = max(0, hi - w)
    return lo, lo + w


def step_plan(ev, t0, W, S):
    """Where the timed steps sit in the decode, and how far the decode runs
    on after them so that one eviction pass is timed.

    Returns (pre, n_main, pass_step): `pre` untimed steps run before the
    warm-up, so that the timed steps centre on the mean steady-state length
    K + B + (P + 1) / 2 of a prompt workload (the cache starts at K + B rows
    after the prompt compression and grows by one row per step until the
    pass at K + B + P); the warm-up and timed steps end at step n_main - 1;
    `pass_step` is the step after which the next pass runs (None without
    eviction).  A cache grown from empty (t0 = 0) starts timing at once, and
    its next pass is the first step that leaves more than K + B rows on a
    period boundary."""
    if not ev:
        return 0, W + S, None
    P, kb = ev["period"], ev["K"] + ev["B"]
    pre = max(0, (P + 1) // 2 - W - S // 2) if t0 else 0
    n_main = pre + W + S
    s = n_main - 1
    while True:
        if (s + 1) % P == 0 and (t0 == 0 and s + 1 > kb or t0 > 0 and s >= n_main - 1):
            if s + 1 >= ev["w"]:
                return pre, n_main, s
        s += 1


def copy_ceiling(dev, nbytes=1 << 30, reps=5):
    """Read + write rate of a plain device copy of nbytes, timed with HIP
    events (the median of reps copies after one warm-up): the machine's copy
    ceiling in this run, for comparison with the attention's read rate."""
    import torch
    x = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    y.copy_(x)
    st = torch.cuda.current_stream()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        y.copy_(x)
        b.record(st)
        b.synchronize()
        ts.append(a.elapsed_time(b))
    del x, y
    ms = sorted(ts)[len(ts) // 2]
    return dict(GBps=round(2 * nbytes / (ms * 1e-3) / 1e9, 1), bytes=2 * nbytes,
                kernel="torch device copy: 1 GiB read + 1 GiB written, median of 5")


def read_ceiling(dev, call_bytes, nbytes=4 << 30, reps=5, n_buf=4, calls=40):
    """Read rates of the library's read probe (kvc_read_probe: the decode
    attention's launch shape and loads without its arithmetic), timed with
    HIP events in the same run: `GBps`, one pass over nbytes (median of reps
    after a warm-up), the part's streaming read rate; `same_size_GBps`,
    `calls` back-to-back reads of the attention call's algorithmic bytes,
    rotating over n_buf buffers as the decode rotates over cache slots (the
    working set exceeds the 256 MB last-level cache), one event pair around
    them: the read rate a kernel of the call's size and launch shape reaches,
    set against the attention call's rate."""
    import torch
    import decode_attention_kvc_amd as kvc
    out = torch.empty(kvc.PROBE_BLOCKS, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream()
    x = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    kvc.kvc_read_probe(x, out)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        kvc.kvc_read_probe(x, out)
        b.record(st)
        b.synchronize()
        ts.append(a.elapsed_time(b))
    del x
    ms = sorted(ts)[len(ts) // 2]
    n1 = max(16, int(call_bytes) // 16 * 16)
    bufs = [torch.ones(n1, dtype=torch.uint8, device=dev) for _ in range(n_buf)]
    for i in range(n_buf):
        kvc.kvc_read_probe(bufs[i], out)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for i in range(calls):
        kvc.kvc_read_probe(bufs[i % n_buf], out)
    b.record(st)
    b.synchronize()
    us_same = a.elapsed_time(b) * 1e3 / calls
    del bufs, out
    return dict(GBps=round(nbytes / (ms * 1e-3) / 1e9, 1), bytes=nbytes,
                same_size_GBps=round(n1 / (us_same * 1e-6) / 1e9, 1), same_size_bytes=n1,
                same_size_us=round(us_same, 2),
                kernel=f"read_probe_kernel (kvc_read_probe): 4 GiB read once, median of {reps}; "
                       f"and {calls} back-to-back reads of the call's bytes over {n_buf} buffers")


def _leg(name, fn, *a, **k):
    """Run one side leg; a Python exception becomes an "error" entry so that
    the headline line is still printed."""
    try:
        r = fn(*a, **k)
        log(f"[bench] {name}: {r}")
        return r
    except Exception as exc:              # noqa: BLE001  (reported, not hidden)
        import traceback
        traceback.print_exc(file=sys.stderr)
        log(f"[bench] {name} leg failed: {type(exc).__name__}: {exc}")
        return {"error": f"{type(exc).__name__}: {exc}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed decode steps (default 20; the Qwen3-4B workload: its 16384 "
                         "generated tokens)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=list(WORKLOADS))
    ap.add_argument("--mode", default=None,
                    choices=["per-layer", "per-layer-interleaved", "grouped"],
                    help="call order (default: the workload's own; per-layer-interleaved "
                         "issues the calls round-robin over the slots, so that no call can "
                         "find its slab in the Infinity Cache)")
    ap.add_argument("--scoring", default="attnv", choices=["attnv", "dkv"],
                    help="eviction scores: observation-window attention (VASE-AttnV) or the "
                         "leverage of Gaussian-sketched [K|V] rows (VASE-DKV)")
    ap.add_argument("--rank", type=int, default=32, choices=[16, 32],
                    help="sketch columns of the VASE-DKV scores")
    ap.add_argument("--no-grouped", action="store_true", help="skip the grouped-mode leg")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip the ragged-batch leg (length mix, per-sequence eviction steps)")
    ap.add_argument("--ragged-only", action="store_true",
                    help="profiling aid: run only the ragged-batch leg and print its result")
    ap.add_argument("--no-xkv", action="store_true",
                    help="skip the cross-layer factorisation / selective reconstruction leg")
    ap.add_argument("--xkv-only", action="store_true",
                    help="profiling aid: run only the cross-layer factorisation leg")
    ap.add_argument("--no-int8", action="store_true",
                    help="skip the range-protected int8 cache leg (decode attention only)")
    ap.add_argument("--protect-frac", type=float, default=0.01,
                    help="fraction of rows per slab the int8 leg keeps in bf16 (largest ranges)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--settle", type=float, default=10.0,
                    help="seconds to wait before the first GPU work (0: none)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (--gpus {args.gpus} "
              "requested); its head/batch sharding is a design note, not built.",
              file=sys.stderr)
        sys.exit(2)

    # A process that freed device memory just before this one (a test run,
    # say) leaves the GPU kernel driver clearing it in the background: decode attention
    # measured ~10% slower over a whole bench run started right after the GPU
    # test suite's process exited (95.0 against 86.5 us per call at the
    # Qwen3-14B shape), and at its usual rate after an 8 s pause.  So the
    # bench waits before its first GPU work.
    if args.settle > 0:
        log(f"[bench] waiting {args.settle:g} s before the first GPU work")
        time.sleep(args.settle)

    import torch
    import kvc_synth
    import decode_attention_kvc_amd as kvc
    from decode_attention_kvc_amd.loop import Decoder

    cfg = dict(WORKLOADS[args.workload])
    if args.mode is None:
        args.mode = cfg.get("mode", "per-layer")
    if cfg["evict"]:
        cfg["evict"] = dict(cfg["evict"], scoring=args.scoring, rank=args.rank)
    dev = "cuda"
    torch.cuda.init()
    L, leaders, nb, hq, hkv, t0 = (cfg[k] for k in ("n_layers", "leaders", "nb", "hq", "hkv", "t0"))
    ev = cfg["evict"]
    n_slots = len(leaders)
    W = args.warmup
    S = args.steps if args.steps is not None else cfg.get("steps", 20)
    if S < 1 or W < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")
    if t0 == 0:
        # A cache grown from empty: the legs built around a prompt cache
        # (ragged prompts, the int8 form of the compressed prompt, the
        # cross-layer factorisation) do not apply.
        args.no_ragged = args.no_int8 = args.no_xkv = True
        if args.ragged_only or args.xkv_only:
            sys.exit("--ragged-only / --xkv-only need a workload with a prompt")
    grouped_leg = not args.no_grouped and args.mode != "grouped" and n_slots < L
    pre, n_main, pass_step = step_plan(ev, t0, W, S)
    n_dec = (pass_step + 1) if pass_step is not None else n_main   # main leg + the run-on
    n_total = n_dec + (S + 1 if grouped_leg else 0)
    if ev and not args.no_ragged and args.workload == "llama3.1-8b-combined":
        # the ragged leg warms up for a full period
        n_total = max(n_total, max(W, ev["period"]) + S + 1)
    if ev:
        n_total = max(n_total, ev["w"])
        steady_cap = ev["K"] + ev["B"] + ev["period"]
    else:
        steady_cap = t0 + n_total
    if args.xkv_only:
        qpool = kvc_synth.queries((L, n_total, nb, hq, 128), device=dev, seed=1)
        knew = kvc_synth.queries((n_total, n_slots, nb, hkv, 128), device=dev, seed=2)
        vnew = kvc_synth.queries((n_total, n_slots, nb, hkv, 128), device=dev, seed=3)
        r = xkv_leg(args, cfg, qpool, knew, vnew, S, warm=W)
        print(json.dumps({"xkv_only": True, "workload": cfg["desc"], "steps": S, "warmup": W,
                          "xkv": r}), flush=True)
        return
    if args.ragged_only:
        if not ev or args.scoring != "attnv":
            sys.exit("--ragged-only needs an eviction workload with window scores")
        qpool = kvc_synth.queries((L, n_total, nb, hq, 128), device=dev, seed=1)
        lsepool = torch.zeros((L, n_total, nb, hq), device=dev)
        knew = kvc_synth.queries((n_total, n_slots, nb, hkv, 128), device=dev, seed=2)
        vnew = kvc_synth.queries((n_total, n_slots, nb, hkv, 128), device=dev, seed=3)
        out = torch.empty((L, nb, hq, 128), device=dev)
        r = ragged_leg(args, cfg, qpool, lsepool, knew, vnew, out, S, warm=W)
        print(json.dumps({"ragged_only": True, "workload": cfg["desc"], "steps": S, "warmup": W,
                          "ragged": r}), flush=True)
        return
    log(f"[bench] {args.workload}: setting up (prompt cache {t0} rows x {n_slots} slots)")

    # ---- inputs (untimed): the prompt cache in a prefill's layout ([t][d]
    # value rows, like the keys), query / append pools
    big = kvc.Cache.empty(n_slots, nb, hkv, t0, device=dev, v_layout="rows") if t0 else None
    prev = None
    for s_ in range(n_slots if t0 else 0):
        Kr, Vr, K32, V32 = kvc_synth.kv_slot(nb, hkv, t0, device=dev, seed=100 + s_,
                                             prev=prev, rho=0.9 if not ev else None,
                                             gap=leaders[1] - leaders[0] if n_slots > 1 else 1)
        big.fill(s_, Kr, Vr)
        prev = (K32, V32) if not ev else None
        del Kr, Vr
    del prev
    qpool = kvc_synth.queries((L, n_total, nb, hq, 128), device=dev, seed=1)
    lsepool = torch.zeros((L, n_total, nb, hq), device=dev)
    if t0:
        knew = kvc_synth.queries((n_total, n_slots, nb, hkv, 128), device=dev, seed=2)
        vnew = kvc_synth.queries((n_total, n_slots, nb, hkv, 128), device=dev, seed=3)
    else:
        # the whole cache is generated rows: they carry the value outliers
        knew, vnew = kvc_synth.append_rows(n_total, n_slots, nb, hkv, device=dev, seed=2)
    out = torch.empty((L, nb, hq, 128), device=dev)
    torch.cuda.synchronize()

    initial_ms = None
    if ev and t0 == 0:
        cache = kvc.Cache.empty(n_slots, nb, hkv, steady_cap, device=dev)
        spare = kvc.Cache.empty(n_slots, nb, hkv, steady_cap, device=dev)
        dec = Decoder(L, leaders, cache, spare, hq, evict=ev, mode=args.mode)
        del big
    elif ev:
        cache = kvc.Cache.empty(n_slots, nb, hkv, steady_cap, device=dev)
        spare = kvc.Cache.empty(n_slots, nb, hkv, steady_cap, device=dev)
        dec = Decoder(L, leaders, big, cache, hq, evict=ev, mode=args.mode)
        q_init = ([kvc_synth.queries((ev["w"], nb, hq, 128), device=dev, seed=50 + i)
                   for i in range(n_slots)] if args.scoring == "attnv" else None)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        dec.initial_pass(q_init)
        b.record()
        torch.cuda.synchronize()
        initial_ms = a.elapsed_time(b)
        log(f"[bench] initial compression {t0} -> {dec.cache.t_len} rows: {initial_ms:.2f} ms")
        dec.spare = spare
        # The prompt's buffers go back to torch's caching allocator, not to
        # the GPU kernel driver (nothing here calls empty_cache): device memory
        # returned to the kernel driver is cleared in the background at ~35 GB/s, and that
        # clear of the 86 GB prompt ran under the timed steps for ~2.4 s,
        # costing 4-5% per attention call (90.7 vs 86.5 us at this shape).
        del big, q_init
    else:
        # no eviction: the prompt's rows enter the decode layout in one copy
        # (kvc_compact with no kept list)
        cache = kvc.Cache.empty(n_slots, nb, hkv, t0 + n_total, device=dev)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for s_ in range(n_slots):
            kvc.kvc_compact(big, s_, None, t0, cache)
        b.record()
        torch.cuda.synchronize()
        cache.t_len = t0
        initial_ms = a.elapsed_time(b)
        log(f"[bench] prompt ingest ({t0} rows x {n_slots} slots, rows -> tiles): "
            f"{initial_ms:.2f} ms")
        del big
        dec = Decoder(L, leaders, cache, None, hq, evict=None, mode=args.mode)

    def run(steps, first, mode, events):
        dec.mode = mode
        if mode == "grouped":
            dec.ws_attn = torch.zeros(max(16, kvc.kvc_decode_attn_ws_bytes(
                dec.cache, max(len(g) for g in dec.groups), hq)), dtype=torch.uint8, device=dev)
        dec.events = [] if events else None
        dec.pass_events = [] if events else None
        n_ev = 0
        for s in range(first, first + steps):
            n_ev += bool(dec.step(s, qpool, lsepool, knew, vnew, out))
        return n_ev

    # ---- pre-roll and warm-up (untimed), then the timed steps.  Python's
    # cyclic collector stays off while GPU work is issued: a full collection
    # stalls the issuing thread for tens of milliseconds, long enough to
    # drain the GPU's queue in the middle of a timed leg.
    gc.collect()
    gc.disable()
    if pre:
        run(pre, 0, args.mode, False)
        log(f"[bench] pre-roll: {pre} steps to {dec.cache.t_len} rows (timed steps centre on the "
            f"mean steady-state length)")
    run(W, pre, args.mode, False)
    torch.cuda.synchronize()
    log(f"[bench] warm-up done ({W} steps), timing {S} steps ({args.mode})")
    t_start = time.perf_counter()
    n_evict = run(S, pre + W, args.mode, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    events = dec.events            # one pair per step around its attention calls
    pass_in = [(a.elapsed_time(b), t, s) for a, b, t, s in dec.pass_events]
    att_ms = [a.elapsed_time(b) for a, b, _, _ in events]
    att_bytes = [step_attn_bytes(dec, args.mode, nb, hq, hkv, t) for (_, _, t, _) in events]
    n_calls = sum(n for _, _, _, n in events)
    att_total_ms = sum(att_ms)
    att_gbps = sum(att_bytes) / (att_total_ms * 1e-3) / 1e9
    avg_launch_us = 1e3 * att_total_ms / n_calls
    t_mean = sum(t for _, _, t, _ in events) / len(events)
    last_step = n_main - 1

    # ---- the eviction pass: timed inside the region, else on the next one
    passes = list(pass_in)
    if ev and not pass_in:
        n_run = pass_step - n_main + 1
        run(n_run, n_main, args.mode, True)
        torch.cuda.synchronize()
        passes = [(a.elapsed_time(b), t, s) for a, b, t, s in dec.pass_events]
        last_step = pass_step
        log(f"[bench] ran on {n_run} untimed steps to the pass after step {pass_step}")
    eviction = None
    if ev:
        if not passes:
            raise RuntimeError("no eviction pass ran")
        t_pass_ms = sum(p[0] for p in passes) / len(passes)
        pass_rows = max(p[1] for p in passes)
        # passes per step: a prompt workload runs one every P steps in its
        # steady state; a cache grown from empty is timed over its whole
        # generation, so the passes it ran are the ones it has
        per_step = (len(pass_in) / S) if t0 == 0 else 1.0 / ev["period"]
        e_bytes = evict_bytes(cfg, pass_rows)
        eviction = dict(ms_per_pass=round(t_pass_ms, 4), rows_at_pass=pass_rows,
                        passes_timed=len(passes), passes_in_timed_steps=len(pass_in),
                        passes_per_step=round(per_step, 6),
                        bytes_per_pass=e_bytes,
                        GBps=round(e_bytes / (t_pass_ms * 1e-3) / 1e9, 1),
                        timing="HIP events around each pass's calls (score + range, select, "
                               "compact on every leader slot)")
    else:
        t_pass_ms, per_step, e_bytes = 0.0, 0.0, 0
    pass_in_ms = sum(p[0] for p in pass_in)
    ms_per_step = (1e3 * wall - pass_in_ms) / S + per_step * t_pass_ms
    tok_s = nb * 1e3 / ms_per_step
    step_bytes = sum(att_bytes) / S + per_step * e_bytes
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"[bench] {S} steps in {wall:.3f} s wall ({len(pass_in)} passes inside); "
        f"attention {att_gbps:.0f} GB/s ({100 * att_gbps / HBM_PEAK_GBPS:.1f}% of peak), avg "
        f"call {avg_launch_us:.1f} us; pass {t_pass_ms:.3f} ms every {ev['period'] if ev else '-'} "
        f"steps -> {ms_per_step:.4f} ms/step, {tok_s:.1f} tok/s")

    grouped = None
    if grouped_leg:
        def grouped_run():
            first = n_dec
            torch.cuda.synchronize()
            g0 = time.perf_counter()
            g_ev = run(S, first, "grouped", True)
            torch.cuda.synchronize()
            gwall = time.perf_counter() - g0
            gev = dec.events
            g_ms = sum(a.elapsed_time(b) for a, b, _, _ in gev)
            g_pass_ms = sum(a.elapsed_time(b) for a, b, _, _ in dec.pass_events)
            g_bytes = sum(step_attn_bytes(dec, "grouped", nb, hq, hkv, t) for (_, _, t, _) in gev)
            g_calls = sum(n for _, _, _, n in gev)
            g_ms_step = (1e3 * gwall - g_pass_ms) / S + per_step * t_pass_ms
            return dict(value=round(nb * 1e3 / g_ms_step, 2), unit="tokens/s",
                        ms_per_step=round(g_ms_step, 4),
                        attention_GBps=round(g_bytes / (g_ms * 1e-3) / 1e9, 1),
                        attention_frac=round(g_bytes / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                        avg_launch_us=round(1e3 * g_ms / g_calls, 2),
                        eviction_passes_in_timed_steps=g_ev,
                        eviction="the main leg's pass time, amortized the same way")
        grouped = _leg("grouped", grouped_run)
        if isinstance(grouped, dict) and "error" not in grouped:
            last_step = n_dec + S - 1
        dec.mode = args.mode

    int8 = None
    if not args.no_int8:
        int8 = _leg("int8", int8_leg, args, cfg, dec, qpool, lsepool, knew, vnew, out, S)

    ragged_res = None
    if (not args.no_ragged and ev and args.scoring == "attnv"
            and args.workload == "llama3.1-8b-combined"):
        log("[bench] ragged leg: setting up")
        ragged_res = _leg("ragged", ragged_leg, args, cfg, qpool, lsepool, knew, vnew, out, S,
                          warm=W)

    xkv_res = None
    if not args.no_xkv and args.workload == "llama3.1-8b-combined":
        log("[bench] xkv leg: factorising the windows")
        dec.spare = None
        xkv_res = _leg("xkv", xkv_leg, args, cfg, qpool, knew, vnew, S, warm=W)

    ceiling = _leg("copy_ceiling", copy_ceiling, dev)
    if isinstance(ceiling, dict) and "GBps" in ceiling:
        ceiling["attention_over_copy"] = round(att_gbps / ceiling["GBps"], 4)
    rceiling = _leg("read_ceiling", read_ceiling, dev, sum(att_bytes) / n_calls)
    if isinstance(rceiling, dict) and "GBps" in rceiling:
        rceiling["attention_over_read"] = round(att_gbps / rceiling["GBps"], 4)
        rceiling["attention_over_same_size"] = round(att_gbps / rceiling["same_size_GBps"], 4)

    if args.copy_calibration:
        # Two plain copies of known size for scaling the memory counters:
        # a 1 GiB runtime blit, and a 512 MiB float32 copy done by a
        # vectorized elementwise kernel (16-byte loads, like the kernels
        # here).
        x = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        y.copy_(x)
        a = torch.zeros(1 << 27, dtype=torch.float32, device=dev)
        c = torch.empty_like(a)
        torch.mul(a, 1.0, out=c)
        torch.cuda.synchronize()
        del x, y, a, c
        log("[bench] copy calibration done: 1 GiB blit, 512 MiB vectorized copy")

    gc.enable()
    cpu = parity = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host (bounded sample)")
        r = _leg("cpu_baseline", cpu_baseline, cfg, dec.cache, qpool, last_step)
        if isinstance(r, tuple):
            cpu, parity = r
        else:
            cpu = parity = r

    traffic, tinfo = load_traffic(args.workload, args.mode, sum(att_bytes) / n_calls)
    res = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": S,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal K/V/Q, 1% x20 value outliers), resident in HBM",
        "config": {
            "workload": cfg["desc"], "name": args.workload, "mode": args.mode,
            "layers": L, "leaders": n_slots, "batch": nb, "q_heads": hq, "kv_heads": hkv,
            "head_dim": 128, "prompt_tokens": t0,
            **({"budget_K": ev["K"], "recent_B": ev["B"], "N_v": ev["N_v"], "window": ev["w"],
                "period": ev["period"], "scoring": ev["scoring"]} if ev else {}),
            **({"sketch_rank": ev["rank"]} if ev and ev["scoring"] == "dkv" else {}),
            "mean_cache_rows": round(t_mean, 1),
            "pre_roll_steps": pre,
        },
        "step_time": ("(wall of the timed steps - the GPU time of passes inside them) / steps "
                      "+ passes per step x the timed pass's GPU time"),
        "decode_ms_per_step": round((1e3 * wall - pass_in_ms) / S, 4),
        "achieved_GBps": round(step_gbps, 1),
        "hbm_frac": round(step_gbps / HBM_PEAK_GBPS, 4),
        "roofline": {
            "kernel": "decode attention call: attn_bf16_kernel (split-K partials) + attn_combine_kernel",
            "bound": "hbm",
            "achieved": round(att_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(att_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_source": None if tinfo is None else tinfo["summary"],
            "avg_launch_us": round(avg_launch_us, 3),
            "launches": n_calls,
            "bytes_per_launch": round(sum(att_bytes) / n_calls),
            "timing": "HIP events around each step's attention calls, on the stream they run on",
        },
        "settle_s": args.settle,
        "copy_ceiling": ceiling,
        "read_ceiling": rceiling,
        "eviction": eviction,
        "eviction_passes_timed": len(passes) if ev else 0,
        "initial_pass_ms": None if initial_ms is None else round(initial_ms, 3),
        "initial_pass": ("prompt compression from the prefill layout (value rows) into the "
                         "tiled decode cache" if ev else "prompt ingest: value rows -> tiles")
        if t0 else None,
        "grouped": grouped,
        "int8": int8,
        "ragged": ragged_res,
        "xkv": xkv_res,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

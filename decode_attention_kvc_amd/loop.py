"""Host schedule of the decode loop over a compressed, cross-layer-shared cache.

Stochastic KV Routing (aitrends.kr article on R-CLA), inference paragraph:
each layer reads the KV of its nearest earlier leader; only leaders append.
VASE summary (gist.science 2606.03928), §2: every `period` steps, when the
cache holds more than K + B rows, an eviction pass (score + range, select,
compact) shrinks every leader slab back to K + B rows; pass r draws its
random keys with seed + r.  The scores are the observation-window attention
(VASE-AttnV, the default) or, with scoring="dkv", the leverage of the
Gaussian-sketched [K | V] rows (VASE-DKV, §2.B), whose projection G is drawn
afresh for every pass and leader: kvc_gaussian_bf16 with key seed + r and
counter (element pair, leader layer, 0xFFFFFFFF).

This module only orders library calls on the current stream; every step of
the computation runs in libkvc's kernels.

Inputs live in pools so that a leader's observation window is a contiguous
slice (no copies):
  qpool    [n_layers][n_steps][nb][Hq][d]   decode queries, cache dtype
  lsepool  [n_layers][n_steps][nb][Hq]      float32, written by attention
  knew, vnew [n_steps][n_slots][nb][Hkv][d] rows each leader appends
"""
import torch

from . import _lib as K


class Decoder:
    def __init__(self, n_layers, leaders, cache, spare, n_q_heads, evict=None,
                 mode="per-layer", record_events=False):
        """cache / spare: two Cache objects of the same shape (ping-pong for
        compaction).  evict: None or dict(K, B, N_v, w, period, seed[,
        scoring="attnv"|"dkv", rank=32]).
        mode: "per-layer" (one call per layer, in layer order), "grouped"
        (one call per leader with all of its followers' queries) or
        "per-layer-interleaved" (one call per layer, issued round-robin over
        the slots -- every leader, then every first follower, ... -- so that
        consecutive calls never read the same slab; each follower still runs
        after its leader has appended)."""
        self.n_layers = n_layers
        self.leaders = list(leaders)
        self.src_layer, self.src_slot = K.kvc_share_map(n_layers, self.leaders)
        self.cache, self.spare = cache, spare
        self.hq = n_q_heads
        self.evict_cfg = evict
        self.mode = mode
        self.round = 1              # pass 0 is the initial compression
        self.last_compaction = None
        dev = cache.k.device
        nb, hkv = cache.nb, cache.n_kv_heads
        # per-layer calls serve one q-layer; grouped calls all followers
        nql = 1 if mode != "grouped" else max(self.src_slot.count(s) for s in range(len(leaders)))
        self.ws_attn = torch.zeros(max(16, K.kvc_decode_attn_ws_bytes(cache, nql, n_q_heads)),
                                   dtype=torch.uint8, device=dev)
        self.groups = [[l for l in range(n_layers) if self.src_slot[l] == s]
                       for s in range(len(leaders))]
        for g in self.groups:
            if g != list(range(g[0], g[0] + len(g))):
                raise ValueError("grouped mode needs each leader's followers to be contiguous")
        self.order = {"per-layer": list(range(n_layers)),
                      "per-layer-interleaved": [g[r] for r in range(max(map(len, self.groups)))
                                                for g in self.groups if r < len(g)]}
        if mode not in ("grouped", *self.order):
            raise ValueError(f"unknown mode {mode!r}")
        self.events = [] if record_events else None
        self._evict_bufs = None

    # ------------------------------------------------------------------ decode
    def step(self, s, qpool, lsepool, knew, vnew, out):
        """Decode step s: leaders append, every layer attends.  out:
        [n_layers][nb][Hq][d] float32 (overwritten)."""
        c = self.cache
        c.t_len += 1
        n_steps = qpool.shape[1]
        nb, hq, d = qpool.shape[2], qpool.shape[3], qpool.shape[4]
        ev = self._ev_begin()
        if self.mode != "grouped":
            for l in self.order[self.mode]:
                slot = self.src_slot[l]
                lead = self.src_layer[l] == l
                K.kvc_decode_attn(c, qpool[l, s], [slot], out[l], lsepool[l, s], self.ws_attn,
                                  k_new=knew[s, slot] if lead else None,
                                  v_new=vnew[s, slot] if lead else None,
                                  append_slot=slot if lead else -1, n_q_heads=hq)
            self._ev_end(ev, c, self.n_layers)
        else:
            for slot, layers in enumerate(self.groups):
                K.kvc_decode_attn(c, qpool[layers[0], s], [slot] * len(layers), out[layers[0]],
                                  lsepool[layers[0], s], self.ws_attn, k_new=knew[s, slot],
                                  v_new=vnew[s, slot], append_slot=slot,
                                  q_layer_stride=n_steps * nb * hq * d,
                                  out_layer_stride=nb * hq * d,
                                  lse_layer_stride=n_steps * nb * hq, n_q_heads=hq)
            self._ev_end(ev, c, len(self.groups))
        e = self.evict_cfg
        if e and (s + 1) % e["period"] == 0 and c.t_len > e["K"] + e["B"]:
            w = e["w"]
            fresh = (s + 1 >= w and (self.last_compaction is None
                                     or self.last_compaction <= s - w + 1 - 1))
            windows = []
            for slot, leader in enumerate(self.leaders):
                q_obs = qpool[leader, s - w + 1:s + 1]
                lse = lsepool[leader, s - w + 1:s + 1] if fresh else None
                windows.append((q_obs, lse))
            self.evict(windows, self.round)
            self.round += 1
            self.last_compaction = s
            return True
        return False

    # ---------------------------------------------------------------- eviction
    def _bufs(self, t_len):
        c = self.cache
        nb, hkv = c.nb, c.n_kv_heads
        b = self._evict_bufs
        if b is None or b["t"] < t_len:
            dev = c.k.device
            e = self.evict_cfg
            t_alloc = max(t_len, c.t_cap)
            b = dict(t=t_alloc,
                     score=torch.empty(nb * hkv * t_alloc, device=dev),
                     g=torch.empty((e.get("rank", 32), 256), dtype=torch.bfloat16, device=dev),
                     dkv_ws=None,
                     rng=torch.empty(nb * hkv * t_alloc, device=dev),
                     kept=torch.empty(nb * hkv * (e["K"] + e["B"]), dtype=torch.int32, device=dev),
                     sel_ws=torch.empty(max(16, K.kvc_select_ws_bytes(nb, hkv, t_alloc)),
                                        dtype=torch.uint8, device=dev),
                     score_ws=torch.zeros(max(16, K.kvc_score_ws_bytes(c, self.hq, e["w"])),
                                          dtype=torch.uint8, device=dev))
            self._evict_bufs = b
        return b

    def evict(self, windows, r):
        """One eviction pass over every leader slot.  windows[slot] =
        (q_obs [w][nb][Hq][d], lse_obs [w][nb][Hq] or None)."""
        e = self.evict_cfg
        c, dst = self.cache, self.spare
        T = c.t_len
        nb, hkv = c.nb, c.n_kv_heads
        n_keep = min(T, e["K"] + e["B"])
        if n_keep == T:
            return
        b = self._bufs(T)
        score = b["score"][: nb * hkv * T]
        rng = b["rng"][: nb * hkv * T]
        kept = b["kept"][: nb * hkv * n_keep]
        dkv = e.get("scoring", "attnv") == "dkv"
        if dkv:
            need = K.kvc_dkv_ws_bytes(c, b["g"].shape[0])
            if b["dkv_ws"] is None or b["dkv_ws"].numel() < need:
                b["dkv_ws"] = torch.empty(need, dtype=torch.uint8, device=c.k.device)
        elif b["score_ws"].numel() < K.kvc_score_ws_bytes(c, self.hq, e["w"]):
            b["score_ws"] = torch.zeros(K.kvc_score_ws_bytes(c, self.hq, e["w"]),
                                        dtype=torch.uint8, device=c.k.device)
        for slot, leader in enumerate(self.leaders):
            if dkv:
                g = b["g"]
                K.kvc_gaussian_bf16(g.numel(), e["seed"] + r, leader, 0xFFFFFFFF, g)
                K.kvc_dkv_score(c, slot, g, score, rng, b["dkv_ws"])
            else:
                q_obs, lse = windows[slot]
                K.kvc_score(c, slot, q_obs, score, rng, lse,
                            None if lse is not None else b["score_ws"])
            K.kvc_select(score, rng, nb, hkv, T, e["K"], e["B"], e["N_v"], e["seed"] + r, leader,
                         kept, b["sel_ws"])
            K.kvc_compact(c, slot, kept, n_keep, dst)
        dst.t_len = n_keep
        self.cache, self.spare = dst, c

    def initial_pass(self, q_obs_by_slot=None):
        """Compress the prompt cache once (pass 0; window scores take two
        passes here, VASE-DKV scores need no queries)."""
        qs = q_obs_by_slot or [None] * len(self.leaders)
        self.evict([(q, None) for q in qs], 0)

    # ------------------------------------------------------------------ events
    def _ev_begin(self):
        if self.events is None:
            return None
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def _ev_end(self, ev, c, n_calls):
        """Close the event pair around one step's attention calls (the
        eviction pass, if any, runs after it)."""
        if ev is None:
            return
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.events.append((ev, e, c.t_len, n_calls))

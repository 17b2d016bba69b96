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

# One-element slot lists for the per-layer calls (built once).
_SLOT_LISTS = [[i] for i in range(256)]


def _one(slot):
    return _SLOT_LISTS[slot] if slot < len(_SLOT_LISTS) else [slot]


def _step_views(qpool, lsepool, knew, vnew, out, s):
    """Per-layer views of step s, made in one call each (indexing the pools
    once per layer costs more host time than the GPU spends on a short
    call)."""
    return (qpool[:, s].unbind(0), lsepool[:, s].unbind(0), out.unbind(0), knew[s].unbind(0),
            vnew[s].unbind(0))


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
        # per-layer calls serve one q-layer; grouped calls all followers.  A
        # prompt cache in a prefill's layout (value rows) is only compressed,
        # never attended: the workspace is sized for the decode cache.
        nql = 1 if mode != "grouped" else max(self.src_slot.count(s) for s in range(len(leaders)))
        att = cache if cache.v_layout == "tiles" or spare is None else spare
        self.ws_attn = torch.zeros(max(16, K.kvc_decode_attn_ws_bytes(att, nql, n_q_heads)),
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
        if evict and evict["period"] < evict["w"]:
            # a pass after step s scores the window of steps s - w + 1 .. s
            raise ValueError(f"the eviction period ({evict['period']}) must be at least the "
                             f"observation window ({evict['w']})")
        self.events = [] if record_events else None
        self.pass_events = [] if record_events else None
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
            qs, ls, outs, kn, vn = _step_views(qpool, lsepool, knew, vnew, out, s)
            for l in self.order[self.mode]:
                slot = self.src_slot[l]
                lead = self.src_layer[l] == l
                K.kvc_decode_attn(c, qs[l], _one(slot), outs[l], ls[l], self.ws_attn,
                                  k_new=kn[slot] if lead else None,
                                  v_new=vn[slot] if lead else None,
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
            if s + 1 < w or s >= n_steps:
                raise ValueError(f"step {s}: the window needs query rows {s - w + 1}..{s} of a "
                                 f"pool of {n_steps}")
            fresh = (s + 1 >= w and (self.last_compaction is None
                                     or self.last_compaction <= s - w + 1 - 1))
            windows = []
            for slot, leader in enumerate(self.leaders):
                q_obs = qpool[leader, s - w + 1:s + 1]
                lse = lsepool[leader, s - w + 1:s + 1] if fresh else None
                windows.append((q_obs, lse))
            ev1 = self._ev_begin()
            t_pass = c.t_len
            self.evict(windows, self.round)
            if ev1 is not None:
                e1 = torch.cuda.Event(enable_timing=True)
                e1.record()
                self.pass_events.append((ev1, e1, t_pass, s))
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


# ---------------------------------------------------------------------------
# Ragged batches
# ---------------------------------------------------------------------------
def ragged_plan(t0, n_steps, evict):
    """The ragged schedule as host bookkeeping: per step the entry and length
    of every sequence during attention ("att_idx", "att_len"), the passes
    ({step: dict(seqs, src, dst, lens, t_len, round, fresh)}), the longest
    length reached ("peak") and the batch entries used ("entries").
    `fresh`: no sequence of the pass was compacted inside its window, so the
    window's log-normalisers from decode attention are valid."""
    nb, ev = len(t0), evict
    kb = ev["K"] + ev["B"] if ev else None
    lens = [min(int(t), kb) for t in t0] if ev else [int(t) for t in t0]
    entry = list(range(nb))
    free = []
    att_idx, att_len, passes = [], [], {}
    last = [-1] * nb                     # step of each sequence's last pass
    peak = max(lens) if lens else 0
    n_entries = nb
    r = 1
    for s in range(n_steps):
        lens = [t + 1 for t in lens]
        peak = max(peak, max(lens))
        att_idx.append(list(entry))
        att_len.append(list(lens))
        if not ev:
            continue
        due = [b for b in range(nb)
               if (s + 1 + ev["phase"][b]) % ev["period"] == 0 and s + 1 >= ev["w"]
               and lens[b] > kb]
        if not due:
            continue
        src = [entry[b] for b in due]
        dst = []
        for b in due:
            if free:
                dst.append(free.pop(0))
            else:
                dst.append(n_entries)
                n_entries += 1
        passes[s] = dict(seqs=due, src=src, dst=dst, lens=[lens[b] for b in due],
                         t_len=max(lens[b] for b in due), round=r,
                         fresh=all(last[b] <= s - ev["w"] for b in due))
        for b, d in zip(due, dst):
            entry[b] = d
            lens[b] = kb
            last[b] = s
        free.extend(src)
        r += 1
    return dict(att_idx=att_idx or [[0] * nb], att_len=att_len or [[0] * nb], passes=passes,
                peak=peak, entries=n_entries, final_len=lens, final_entry=entry)


class RaggedDecoder:
    """Decode loop of a ragged batch: every sequence has its own length and
    runs its eviction passes on its own steps.

    VASE summary (gist.science 2606.03928), §2 gives the periodic pass per
    sequence.  Sequence b has a phase p_b and is due after step s when
    (s + 1 + p_b) is a multiple of the period, it has decoded at least w
    steps, and it holds more than K + B rows.  The sequences due after one
    step form one pass (pass r uses seed + r, the prompt compression being
    pass 0); the Philox counter's batch word is the sequence index.

    Every sequence lives in one batch entry of `cache`, which holds a few
    more entries than sequences: a pass compacts each due sequence into a
    free entry and frees the one it leaves (no second cache, and sequences
    that are not due are not touched).  Because every sequence appends one
    row per step, the whole schedule (lengths, due sets, entries) is host
    bookkeeping fixed by the prompt lengths; it is planned here once and its
    per-step device arrays are uploaded once, so a step only launches
    kernels.  A pass's calls address the due sequences; their window
    queries and log-normalisers are read from the pools' own [w][nb] slices
    through the due sequences' indices (kvc_score_seq).
    """

    def __init__(self, n_layers, leaders, cache, n_q_heads, t0, n_steps, evict=None,
                 mode="grouped", record_events=False):
        """record_events: keep HIP event pairs around each step's attention
        calls (self.events: (start, end, step, n_calls)) and each eviction
        pass (self.pass_events: (start, end, step, n_sequences))."""
        self.events = [] if record_events else None
        self.pass_events = [] if record_events else None
        self.n_layers = n_layers
        self.leaders = list(leaders)
        self.src_layer, self.src_slot = K.kvc_share_map(n_layers, self.leaders)
        self.cache = cache
        self.hq = n_q_heads
        self.ev = evict
        self.mode = mode
        self.nb = nb = len(t0)
        self.t0 = [int(x) for x in t0]
        self.groups = [[l for l in range(n_layers) if self.src_slot[l] == s]
                       for s in range(len(leaders))]
        if mode == "grouped":
            for g in self.groups:
                if g != list(range(g[0], g[0] + len(g))):
                    raise ValueError("grouped mode needs each leader's followers to be contiguous")
        elif mode != "per-layer":
            raise ValueError(f"unknown mode {mode!r}")
        dev = cache.k.device
        plan = ragged_plan(self.t0, n_steps, evict)
        if max(plan["peak"], 1) > cache.t_cap:
            raise ValueError(f"the schedule reaches {plan['peak']} rows; t_cap is {cache.t_cap}")
        if plan["entries"] > cache.nb_cap:
            raise ValueError(f"the schedule needs {plan['entries']} batch entries; "
                             f"the cache has {cache.nb_cap}")
        self.plan = plan
        # per-step entries and lengths, one upload
        self.att_idx = torch.tensor(plan["att_idx"], dtype=torch.int32, device=dev)
        self.att_len = torch.tensor(plan["att_len"], dtype=torch.int32, device=dev)
        # A pass addresses the due sequences only (their entries and
        # lengths); their window queries and log-normalisers stay in the
        # pools' [w][nb] slices, which kvc_score_seq reads through the due
        # sequences' indices: no gather runs between the library calls.
        self.passes = {}
        for s, p in plan["passes"].items():
            arr = torch.tensor([p["seqs"], p["src"], p["dst"], p["lens"]], dtype=torch.int32,
                               device=dev)
            self.passes[s] = dict(p, seqs_d=arr[0], src_d=arr[1], dst_d=arr[2], lens_d=arr[3])
        self.prompt_len = torch.tensor(self.t0, dtype=torch.int32, device=dev)
        self.seq_ids = torch.arange(nb, dtype=torch.int32, device=dev)
        nql = 1 if mode != "grouped" else max(len(g) for g in self.groups)
        self.ws_attn = torch.zeros(max(16, K.kvc_decode_attn_ws_bytes(
            cache.seqs(self.seq_ids, self.prompt_len, t_len=cache.t_cap), nql, n_q_heads)),
            dtype=torch.uint8, device=dev)
        self._ebufs = None

    def view(self, s):
        """The cache as decode step s addresses it."""
        return self.cache.seqs(self.att_idx[s], self.att_len[s],
                               t_len=int(max(self.plan["att_len"][s])))

    # ------------------------------------------------------------------ decode
    def step(self, s, qpool, lsepool, knew, vnew, out):
        """Decode step s: every sequence appends (leaders) and attends, then
        the sequences due run their eviction pass.  Returns True if a pass
        ran."""
        c = self.view(s)
        n_steps = qpool.shape[1]
        nb, hq, d = qpool.shape[2], qpool.shape[3], qpool.shape[4]
        ev0 = self._event()
        if self.mode == "per-layer":
            qs, ls, outs, kn, vn = _step_views(qpool, lsepool, knew, vnew, out, s)
            for l in range(self.n_layers):
                slot = self.src_slot[l]
                lead = self.src_layer[l] == l
                K.kvc_decode_attn(c, qs[l], _one(slot), outs[l], ls[l], self.ws_attn,
                                  k_new=kn[slot] if lead else None,
                                  v_new=vn[slot] if lead else None,
                                  append_slot=slot if lead else -1, n_q_heads=hq)
        else:
            for slot, layers in enumerate(self.groups):
                K.kvc_decode_attn(c, qpool[layers[0], s], [slot] * len(layers), out[layers[0]],
                                  lsepool[layers[0], s], self.ws_attn, k_new=knew[s, slot],
                                  v_new=vnew[s, slot], append_slot=slot,
                                  q_layer_stride=n_steps * nb * hq * d,
                                  out_layer_stride=nb * hq * d,
                                  lse_layer_stride=n_steps * nb * hq, n_q_heads=hq)
        if ev0 is not None:
            self.events.append((ev0, self._event(), s,
                                self.n_layers if self.mode == "per-layer" else len(self.groups)))
        p = self.passes.get(s)
        if p is None:
            return False
        ev1 = self._event()
        w = self.ev["w"]
        if s + 1 < w or s >= n_steps:
            raise ValueError(f"step {s}: the window needs query rows {s - w + 1}..{s} of a "
                             f"pool of {n_steps}")
        windows = []
        for leader in self.leaders:
            q_obs = qpool[leader, s - w + 1:s + 1]
            lse = lsepool[leader, s - w + 1:s + 1] if p["fresh"] else None
            windows.append((q_obs, lse))
        src = self.cache.seqs(p["src_d"], p["lens_d"], t_len=p["t_len"])
        dst = self.cache.seqs(p["dst_d"], None, t_len=self.ev["K"] + self.ev["B"])
        self._pass(src, dst, windows, p["seqs_d"], p["round"])
        if ev1 is not None:
            self.pass_events.append((ev1, self._event(), s, len(p["seqs"])))
        return True

    def _event(self):
        if self.events is None:
            return None
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    # ---------------------------------------------------------------- eviction
    def _bufs(self, src):
        """Eviction buffers for a pass over the sequences of `src` (grown on
        demand, kept between passes)."""
        n, t, hkv = src.nb, src.t_len, src.n_kv_heads
        e, dev = self.ev, src.k.device
        b = self._ebufs
        if b is None or b["n"] < n or b["t"] < t:
            n, t = max(n, b["n"] if b else 0), max(t, b["t"] if b else 0)
            b = dict(n=n, t=t, score=torch.empty(n * hkv * t, device=dev),
                     rng=torch.empty(n * hkv * t, device=dev),
                     kept=torch.empty(n * hkv * (e["K"] + e["B"]), dtype=torch.int32, device=dev),
                     sel_ws=torch.empty(max(16, K.kvc_select_ws_bytes(n, hkv, t)),
                                        dtype=torch.uint8, device=dev),
                     score_ws=torch.zeros(16, dtype=torch.uint8, device=dev))
            self._ebufs = b
        key = (n, src.t_cap)
        need = b.get(key)
        if need is None:
            need = b[key] = K.kvc_score_ws_bytes(src, self.hq, e["w"])
        if b["score_ws"].numel() < need:
            b["score_ws"] = torch.zeros(need, dtype=torch.uint8, device=dev)
        return b

    def _pass(self, src, dst, windows, seq_ids, r):
        """One eviction pass over the sequences of `src` (moved to the entries
        of `dst`), every leader slot."""
        e = self.ev
        n, hkv, T = src.nb, src.n_kv_heads, src.t_len
        n_keep = min(T, e["K"] + e["B"])
        b = self._bufs(src)
        score = b["score"][: n * hkv * T]
        rng = b["rng"][: n * hkv * T]
        kept = b["kept"][: n * hkv * n_keep]
        for slot, leader in enumerate(self.leaders):
            q_obs, lse = windows[slot]
            K.kvc_score_seq(src, slot, q_obs, seq_ids, score, rng, lse,
                            None if lse is not None else b["score_ws"])
            K.kvc_select_seq(score, rng, n, hkv, T, src.seq_len, seq_ids, e["K"], e["B"], e["N_v"],
                             e["seed"] + r, leader, kept, b["sel_ws"])
            K.kvc_compact(src, slot, kept, n_keep, dst)

    def initial_pass(self, prompt, q_obs_by_slot):
        """Pass 0: compress each sequence's prompt (entry b of `prompt`, t0[b]
        rows) into its entry of the decode cache (min(t0[b], K + B) rows;
        shorter prompts are copied whole)."""
        src = prompt.seqs(None, self.prompt_len, t_len=max(self.t0))
        dst = self.cache.seqs(self.seq_ids, None, t_len=self.ev["K"] + self.ev["B"])
        self._pass(src, dst, [(q, None) for q in q_obs_by_slot], self.seq_ids, 0)

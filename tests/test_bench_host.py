"""Host-side pieces of the benchmark and the synthetic inputs (CPU only):
the single-GPU refusal, the workload table, the algorithmic byte counts the
roofline figures divide by, and the value-outlier recipe of generated rows."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import kvc_synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("name", list(bench.WORKLOADS))
def test_workload_table(name):
    w = bench.WORKLOADS[name]
    leaders = w["leaders"]
    assert leaders[0] == 0 and leaders == sorted(set(leaders)) and leaders[-1] < w["n_layers"]
    assert w["hq"] % w["hkv"] == 0
    e = w["evict"]
    if e:
        assert 0 <= e["N_v"] <= e["K"] and e["B"] >= 0 and e["period"] >= e["w"] >= 1


def test_attention_bytes_by_hand():
    # nb 2, 8 query / 2 KV heads, 10 rows: K and V (2 * 2 slabs * 10 rows *
    # 256 B), queries (2 * 8 * 256 B), float32 out + lse (2 * 8 * 129 * 4 B),
    # and a leader's appended K and V rows (2 * 2 slabs * 256 B)
    kv, q, out, app = 2 * 2 * 2 * 10 * 256, 2 * 8 * 256, 2 * 8 * 129 * 4, 2 * 2 * 2 * 256
    assert bench.attn_bytes(2, 8, 2, 10, 1, False) == kv + q + out
    assert bench.attn_bytes(2, 8, 2, 10, 1, True) == kv + q + out + app
    # a grouped call serving 3 q-layers reads the slab once
    assert bench.attn_bytes(2, 8, 2, 10, 3, True) == kv + 3 * q + 3 * out + app


def test_eviction_bytes_by_hand():
    cfg = dict(nb=2, hkv=2, leaders=[0, 3],
               evict=dict(K=6, B=2, N_v=1, w=2, period=4, seed=0))
    slabs = 2 * 2 * 2
    t = 12
    # K + V read once (2 * t * 256), score and range written and read
    # (2 * 4 * t * 2), kept indices (4 * 8), kept rows read and written
    # (2 * 2 * 8 * 256)
    per_slab = 2 * t * 256 + 2 * 4 * t * 2 + 4 * 8 + 2 * 2 * 8 * 256
    assert bench.evict_bytes(cfg, t) == slabs * per_slab


def test_append_rows_outliers():
    n, slots, nb, hkv = 250, 3, 2, 4
    k1, v1 = kvc_synth.append_rows(n, slots, nb, hkv, dtype=torch.float32, seed=9)
    k0, v0 = kvc_synth.append_rows(n, slots, nb, hkv, dtype=torch.float32, seed=9,
                                   outlier_frac=0.0)
    assert torch.equal(k1, k0)                       # keys carry no outliers
    changed = (v1 != v0).any(dim=-1)                 # [n][slots][nb][hkv]
    per_seq = changed.sum(dim=0)
    assert torch.all(per_seq == round(0.01 * n))     # round(1% of the rows) each
    assert torch.equal(v1[changed], 20.0 * v0[changed])
    assert torch.equal(v1[~changed], v0[~changed])


@pytest.mark.parametrize("W,S", [(5, 20), (2, 1), (0, 1), (3, 256)])
@pytest.mark.parametrize("name", list(bench.WORKLOADS))
def test_step_plan_and_windows(name, W, S):
    """The steps the bench runs and the window slices it takes stay inside
    the query pool, a pass is always timed, and the timed steps of a prompt
    workload centre on the steady state's mean length."""
    w_ = bench.WORKLOADS[name]
    ev, t0 = w_["evict"], w_["t0"]
    pre, n_main, pass_step = bench.step_plan(ev, t0, W, S)
    assert n_main == pre + W + S
    if ev is None:
        assert pass_step is None and pre == 0
        return
    P, kb = ev["period"], ev["K"] + ev["B"]
    assert pass_step >= n_main - 1 and (pass_step + 1) % P == 0
    assert pass_step + 1 >= ev["w"]
    if t0:
        assert pass_step - (n_main - 1) < P            # the next pass, not a later one
        first = pre + W                                  # rows = K + B + step + 1
        if S < P - W:
            mid = kb + first + 1 + (S - 1) / 2
            assert abs(mid - (kb + (P + 1) / 2)) <= 1.0
    else:
        assert pass_step + 1 > kb
    # every window the bench slices exists and has w rows
    n_pool = pass_step + 1
    for s in range(0, n_pool):
        lo, hi = bench.window_rows(s, ev["w"], max(n_pool, ev["w"]))
        assert 0 <= lo and hi - lo == ev["w"] and hi <= max(n_pool, ev["w"])
        if s + 1 >= ev["w"]:
            assert hi == s + 1                           # the w rows ending at step s


def test_window_rows_driver_command():
    # --steps 20 --warmup 5 with w = 32: the last step is 24; the slice used
    # to start at -7 (an empty slice); now it is the pool's first 32 rows
    assert bench.window_rows(24, 32, 400) == (0, 32)
    assert bench.window_rows(255, 32, 400) == (224, 256)
    assert bench.window_rows(1, 32, 33) == (0, 32)
    with pytest.raises(ValueError):
        bench.window_rows(5, 32, 31)


def test_decoder_rejects_period_shorter_than_window():
    from decode_attention_kvc_amd.loop import Decoder
    import decode_attention_kvc_amd as kvc
    c = kvc.Cache.empty(1, 1, 2, 64, dtype=torch.float32, device="cpu")
    with pytest.raises(ValueError, match="period"):
        Decoder(2, [0], c, c, 8, evict=dict(K=8, B=2, N_v=1, w=32, period=16, seed=0))

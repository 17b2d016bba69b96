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

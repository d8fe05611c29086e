"""The bench's contract: its refusal of several GPUs, the algorithmic bytes its
HBM roofline divides by, and (on a GPU) the fields of its one JSON line.

The byte count is pinned by a closed form written from the workload's shape
alone: per sequence, every key up to the last query's position is visible
(causal block at the end of the context) unless a window cuts the span, and
each visible key moves K and V codes for every KV head.
"""
import json
import os
import subprocess
import sys

import pytest

from paged_quantized_kv_ra_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("kv, e, scale_bytes", [("e4m3", 1, 0), ("int8", 1, 0), ("f16", 2, 0), ("int8_tok", 1, 4)])
def test_algorithmic_bytes_closed_form(kv, e, scale_bytes):
    ctx, q_len, hq, hkv, d = [300, 17, 1000], [5, 1, 16], 8, 2, 64
    w = W.build("t", 3, ctx=ctx, q_len=q_len, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, kv_dtype=kv)
    t = sum(q_len)
    kv_bytes = sum(ctx) * 2 * hkv * (d * e + scale_bytes)
    table = 4 * sum((c + 15) // 16 for c in ctx)
    q_bytes = t * hq * d * 2
    out_bytes = t * hq * d * 2 + t * hq * 4
    assert bench.algorithmic_bytes(w) == kv_bytes + table + q_bytes + out_bytes


def test_algorithmic_bytes_window_and_sinks():
    # one sequence of 1000 keys, 16 queries at 984..999, window 100, 4 sinks:
    # keys 885..999 (115) are in some query's window, plus sinks 0..3
    w = W.build("t", 4, ctx=[1000], q_len=[16], num_q_heads=4, num_kv_heads=1, head_dim=64,
                kv_dtype="e4m3", window_left=100, num_sinks=4)
    kv_bytes = (115 + 4) * 2 * 1 * 64
    table = 4 * ((1000 + 15) // 16)
    q_bytes = 16 * 4 * 64 * 2
    assert bench.algorithmic_bytes(w) == kv_bytes + table + q_bytes + q_bytes + 16 * 4 * 4


def test_unique_bytes_count_shared_prefix_pages_once():
    # 3 sequences of 100 keys whose first 64 keys (4 pages) share physical
    # pages: 4 shared + 3 x 3 private pages hold all visible keys
    w = W.build("t", 5, ctx=[100] * 3, q_len=1, num_q_heads=2, num_kv_heads=1, head_dim=64, kv_dtype="int8",
                shared_prefix_tokens=64)
    per_token = 2 * 1 * 64
    base = bench.algorithmic_bytes(w) - 300 * per_token
    assert bench.algorithmic_bytes(w, unique=True) == base + (4 + 3 * 3) * 16 * per_token


@pytest.mark.gpu
def test_bench_json_line():
    print("bench.py --workload tiny_decode --steps 5 --warmup 2 --cpu-seconds 0.5", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "tiny_decode",
                        "--steps", "5", "--warmup", "2", "--cpu-seconds", "0.5"],
                       capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    j = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in j, key
    assert j["n_gpus"] == 1 and j["steps"] == 5 and j["warmup"] == 2 and j["value"] > 0
    assert j["config"]["workload"] == "tiny_decode_ctx256_f16"
    roof = j["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert roof["achieved"] > 0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    for k in ("attn_us_p10", "attn_us_median", "attn_us_p90"):
        assert roof[k] > 0, k
    assert roof["attn_us_p10"] <= roof["attn_us_median"] <= roof["attn_us_p90"]
    assert "hbm_gbs" in roof
    st = j["step_us_percentiles"]
    assert 0 < st["p10"] <= st["median"] <= st["p90"]
    cb = j["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert len(cb["runs_value"]) == 3 and sorted(cb["runs_value"])[1] == round(cb["value"], 1)
    one = cb["single_thread"]
    assert one["cores"] == 1 and one["value"] > 0 and len(one["runs_value"]) == 3

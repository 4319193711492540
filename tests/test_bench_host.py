"""Host logic of bench.py (CPU only).

* Row counting: the rows of each item (live source budgets that can still execute, plus the
  reference row) equal an independent set-based reachability count.
* Algorithmic work of the Llama-3-8B 32K solve: weight, KV and state bytes and the GEMM and
  attention FLOPs recomputed by hand from the shapes and the reachable rows, and checked
  against the per-solve figures worked out for this configuration (13.959 GB of weights,
  4.295 GB of KV, 1.684 TFLOP of GEMM, 2.033 TFLOP of attention).
* --gpus above 1 exits with a message (one GPU only).
* The CPU baseline stops the oracle at an item boundary and scales by the finished items'
  FLOP share.
* The profile summary scales the FETCH_SIZE / WRITE_SIZE counters by the copy calibration.
"""
import csv
import json
import os
import subprocess
import sys
import types

import pytest

import bench
from oracle import knapspec_oracle as ko
from workloads import WORKLOADS, scaled, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _weights(wl, ctx):
    lat = wl.latency
    t = ko.item_latencies(wl.shape.n_layers, ctx, lat.attn_base, lat.attn_per_token, lat.mlp)
    return [int(x) for x in ko.item_weights(t, wl.n_budgets)]


def _rows_by_sets(w, B):
    reach, rows = {0}, []
    for wi in w:
        rows.append(len([s for s in reach if s + wi <= B - 1]) + 1)
        reach = reach | {s + wi for s in reach if s + wi <= B - 1}
    return rows


@pytest.mark.parametrize("name", ["tiny", "qwen3_1p7b_4k", "llama3_8b_32k", "llama3_70b_32k"])
def test_item_rows_equal_reachability(name):
    wl = WORKLOADS[name]
    w = _weights(wl, wl.ctx)
    rows, live = bench.item_rows(w, wl.n_budgets)
    assert rows == _rows_by_sets(w, wl.n_budgets)
    assert all(1 <= v <= wl.n_budgets for v in live)


def test_algorithmic_work_llama3_8b_32k():
    wl = WORKLOADS["llama3_8b_32k"]
    s = wl.shape
    ctx = 32768
    w = _weights(wl, ctx)
    assert (w[0], w[1], sum(w)) == (3, 5, 256)
    cls, tot = bench.algorithmic_work(wl, [w], [ctx])
    d, ff, dh, hq, hkv, L = s.d_model, s.d_ff, s.head_dim, s.n_q_heads, s.n_kv_heads, s.n_layers
    nqkv = (hq + 2 * hkv) * dh
    # weights: q|k|v, O, gate|up, down per layer, bf16
    wb = L * 2 * (nqkv * d + d * hq * dh + 2 * ff * d + d * ff)
    assert tot["weight_bytes"] == wb
    assert tot["kv_bytes"] == L * 2 * hkv * ctx * dh * 2
    rows = _rows_by_sets(w, wl.n_budgets)
    gemm = sum(2.0 * R * (nqkv * d + d * hq * dh) for R in rows[0::2]) + \
        sum(2.0 * R * 3 * ff * d for R in rows[1::2])
    attn = sum(4.0 * R * hq * ctx * dh for R in rows[0::2])
    got_gemm = sum(cls[k]["flops"] for k in ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down"))
    assert got_gemm == pytest.approx(gemm, rel=1e-12)
    assert cls["attention"]["flops"] == pytest.approx(attn, rel=1e-12)
    # the per-solve figures of this configuration, to their printed precision
    assert round(tot["weight_bytes"] / 1e9, 3) == 13.959
    assert round(tot["kv_bytes"] / 1e9, 3) == 4.295
    # state: every source row (and the reference row) read, every live budget written, fp32
    live, reach = [], {0}
    for wi in w:
        reach = reach | {x + wi for x in reach if x + wi <= wl.n_budgets - 1}
        live.append(len(reach))
    assert tot["state_bytes"] == sum((R + V) * d * 4 for R, V in zip(rows, live))
    assert round(got_gemm / 1e12, 3) == 1.684
    assert round(cls["attention"]["flops"] / 1e12, 3) == 2.033
    assert tot["total_bytes"] == tot["weight_bytes"] + tot["kv_bytes"] + tot["state_bytes"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _small_problem():
    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=3, d_model=256, n_q_heads=4,
                n_kv_heads=2, head_dim=64, d_ff=512, n_budgets=24, name="bench_host_t")
    ctx = 96
    prob = types.SimpleNamespace(
        ctxs=[ctx],
        host_layers=[synth.layer_weights(wl, l, 0) for l in range(wl.shape.n_layers)],
        host_kv=[[synth.kv_cache(wl, l, 0, ctx, 0) for l in range(wl.shape.n_layers)]],
        host_x0=[synth.x0(wl, 0, 0)])
    return wl, prob


def test_cpu_baseline_whole_solve_and_early_stop():
    wl, prob = _small_problem()
    full = bench.cpu_baseline(wl, prob, 1000, lambda *a: None, seconds=1e9, repeats=3,
                              seconds_1t=1e9)
    assert full["kind"] == "oracle" and full["value"] > 0 and full["cores"] >= 1
    assert "[6, 6, 6] of 6 items" in full["sample"] and "median of 3" in full["sample"]
    assert len(full["repeats"]) == 3 and sorted(full["repeats"])[1] == pytest.approx(full["value"], rel=1e-5)
    assert full["value_1_thread"] > 0 and "first 6 items" in full["sample_1_thread"]
    assert "(FLOP share 1.0000)" in full["sample_1_thread"]
    assert full["cpu_model"] and full["blas"]
    part = bench.cpu_baseline(wl, prob, 1000, lambda *a: None, seconds=0.0, repeats=1,
                              seconds_1t=0.0)
    # stopped when item 1 starts: only item 0 (the first Attention item) was timed
    assert "[1] of 6 items" in part["sample"] and "first 1 items" in part["sample_1_thread"]
    assert part["value"] > 0


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)


def test_summarize_profiles_scales_counters(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    k_attn, k_gemm = "attn_mfma_kernel(ks::AttnArgs)", "gemm_lds_kernel<4, 4, 3>(ks::GemmArgs)"
    _write_csv(str(tmp_path / "stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"],
               [[k_gemm, 2, 100000, 50000, 40.0], [k_attn, 2, 150000, 75000, 60.0]])
    hdr = ["Kernel_Name", "Dispatch_Id", "Counter_Name", "Counter_Value"]
    # two dispatches of the dominant kernel: 1000 and 3000 KiB fetched; 500 KiB written
    _write_csv(str(tmp_path / "fetch" / "a" / "run_counter_collection.csv"), hdr,
               [[k_attn, 1, "FETCH_SIZE", 1000], [k_attn, 2, "FETCH_SIZE", 3000],
                [k_gemm, 3, "FETCH_SIZE", 7]])
    _write_csv(str(tmp_path / "write" / "a" / "run_counter_collection.csv"), hdr,
               [[k_attn, 1, "WRITE_SIZE", 500], [k_attn, 2, "WRITE_SIZE", 500]])
    # a 1 MiB copy reads as 512 KiB fetched (factor 2) and 1024 KiB written (factor 1)
    _write_csv(str(tmp_path / "cfetch" / "a" / "run_counter_collection.csv"), hdr,
               [["copy", 1, "FETCH_SIZE", 512], ["copy", 2, "FETCH_SIZE", 4]])
    _write_csv(str(tmp_path / "cwrite" / "a" / "run_counter_collection.csv"), hdr,
               [["copy", 1, "WRITE_SIZE", 1024]])
    args = types.SimpleNamespace(
        stats=str(tmp_path / "stats.csv"), fetch=str(tmp_path / "fetch"),
        write=str(tmp_path / "write"), copy_fetch=str(tmp_path / "cfetch"),
        copy_write=str(tmp_path / "cwrite"), copy_bytes=1 << 20, workload="unit",
        commands="cmd one;;cmd two")
    bench.summarize_profiles(args)
    t = json.load(open(tmp_path / "profiles" / "traffic_unit.json"))
    assert t["kernel"] == k_attn
    assert t["copy_factor_fetch"] == pytest.approx(2.0)
    assert t["copy_factor_write"] == pytest.approx(1.0)
    assert t["fetch_bytes_per_launch"] == pytest.approx(2000 * 1024 * 2.0)
    assert t["write_bytes_per_launch"] == pytest.approx(500 * 1024 * 1.0)
    assert t["source_sha"] == bench.kernel_source_sha()
    md = open(tmp_path / "profiles" / "attention_unit.md").read()
    assert "cmd one\ncmd two" in md and "| 2 | 75.0 | 60.0 | 4.10 | 0.51 |" in md

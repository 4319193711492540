#!/usr/bin/env python3
"""Benchmark: KnapSpec DP solves/s on one MI355X for the Llama-3-8B-shaped 32K-context workload.

One step = one full knapspec_solve (all 64 items x 256 budgets, attention over 32768 cached
positions, cosine/select, D2H of the per-budget results and the host TPT grid) on inputs
already resident in HBM.  Prints ONE JSON line on stdout; progress goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KnapSpec DP solves/sec + achieved HBM GB/s, Llama-3-8B-shape ctx 32K"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense; f32 path runs on the vector ALUs


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def item_rows(w, B, beam=1):
    """Rows of each item's GEMM per sequence: the source states (budgets s with s + w_i <= B-1,
    up to ``beam`` states each -- the number of distinct subsets of weight s, capped), plus the
    reference row, and the live states after the item (same bookkeeping as the library;
    measurement only)."""
    cnt = [0] * B
    cnt[0] = 1
    rows, live = [], []
    for wi in w:
        src = sum(cnt[s] for s in range(B) if s + wi <= B - 1)
        rows.append(src + 1)
        cnt = [min(beam, cnt[b] + (cnt[b - wi] if b >= wi else 0)) for b in range(B)]
        live.append(sum(cnt))
    return rows, live


def algorithmic_work(wl, w_per_seq, ctxs, window=1, vocab=0, beam=1):
    """Minimum HBM bytes and FLOPs of one solve, per kernel class and in total.

    Per item: its weight matrix once; for Attention items the sequence's K and V cache once;
    the activation rows it reads and the rows it writes once; and for the state a read of every
    source row plus a write of every live budget (fp32).  With an r-token window every
    budget row is r token rows; with an LM head of ``vocab`` rows the acceptance estimate
    reads the head once and the (budgets + 1) x r final rows."""
    s = wl.shape
    eb = s.elem_bytes
    d, ff, dh, hq, hkv = s.d_model, s.d_ff, s.head_dim, s.n_q_heads, s.n_kv_heads
    qd, nqkv = hq * dh, (hq + 2 * hkv) * dh
    cls = {k: {"bytes": 0.0, "flops": 0.0, "launches": 0} for k in
           ("gemm_qkv", "qkv_rope", "attention", "combine", "gemm_o", "gemm_gate_up",
            "gemm_down", "select", "lm_head")}
    L2 = 2 * s.n_layers
    per_item_rows = []
    for q, w in enumerate(w_per_seq):
        rows, live = item_rows(list(w), wl.n_budgets, beam)
        per_item_rows.append(([x * window for x in rows], [x * window for x in live]))
    for i in range(L2):
        R = sum(pr[0][i] for pr in per_item_rows)
        V = sum(pr[1][i] for pr in per_item_rows)
        if i % 2 == 0:
            c = cls["gemm_qkv"]
            c["bytes"] += nqkv * d * eb + R * d * eb + R * nqkv * 4
            c["flops"] += 2.0 * R * nqkv * d
            c["launches"] += 1
            c = cls["qkv_rope"]
            c["bytes"] += R * nqkv * 4 + R * (qd * eb + 2 * hkv * dh * 4)
            c["launches"] += 1
            c = cls["attention"]
            for q, pr in enumerate(per_item_rows):
                Rq = pr[0][i]
                c["bytes"] += 2 * hkv * ctxs[q] * dh * eb + Rq * qd * eb + Rq * qd * 4
                c["flops"] += 4.0 * Rq * hq * ctxs[q] * dh
            c["launches"] += 1
            c = cls["combine"]
            c["bytes"] += R * qd * 4 + R * qd * eb
            c["launches"] += 1
            c = cls["gemm_o"]
            c["bytes"] += d * qd * eb + R * qd * eb + R * d * 4
            c["flops"] += 2.0 * R * d * qd
            c["launches"] += 1
        else:
            c = cls["gemm_gate_up"]
            c["bytes"] += 2 * ff * d * eb + R * d * eb + R * ff * eb
            c["flops"] += 2.0 * R * 2 * ff * d
            c["launches"] += 1
            c = cls["gemm_down"]
            c["bytes"] += d * ff * eb + R * ff * eb + R * d * 4
            c["flops"] += 2.0 * R * d * ff
            c["launches"] += 1
        c = cls["select"]
        c["bytes"] += (R + V) * d * 4
        c["launches"] += 1
    if vocab:
        c = cls["lm_head"]
        Rlm = len(w_per_seq) * (wl.n_budgets + 1) * window
        c["bytes"] += vocab * d * eb + Rlm * d * eb
        c["flops"] += 2.0 * Rlm * vocab * d
        c["launches"] += 1
    w_bytes = s.n_layers * (s.attn_weight_bytes() + s.mlp_weight_bytes()) + vocab * d * eb
    kv_bytes = sum(2 * hkv * c_ * dh * eb * s.n_layers for c_ in ctxs)
    state_bytes = cls["select"]["bytes"] + (cls["lm_head"]["bytes"] - vocab * d * eb)
    total_bytes = w_bytes + kv_bytes + state_bytes
    total_flops = sum(cls[k]["flops"] for k in cls)
    return cls, {"weight_bytes": w_bytes, "kv_bytes": kv_bytes, "state_bytes": state_bytes,
                 "total_bytes": total_bytes, "total_flops": total_flops,
                 "mean_rows": sum(sum(pr[0]) for pr in per_item_rows) / L2}


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "draft_layer_selection_amd", "csrc")


def kernel_source_sha() -> str:
    """Hash of the HIP/C++ sources: counter figures taken on other sources are stale."""
    import hashlib

    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".cpp", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def copy_calibration(nbytes: int):
    """A plain device copy of known size (torch's copy kernel), for scaling the FETCH_SIZE /
    WRITE_SIZE counters to bytes."""
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": src.numel() * 4}))


def _pmc_per_kernel(path_dir, counter):
    """{kernel name: [per-dispatch counter values]} from a rocprofv3 --pmc csv directory."""
    import csv
    import glob

    out = {}
    for f in glob.glob(os.path.join(path_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            out.setdefault(key, 0.0)
            out[key] += float(r["Counter_Value"])
    per = {}
    for (name, _), v in out.items():
        per.setdefault(name, []).append(v)
    return per


def kernel_tag(name: str) -> str:
    """Short file-name tag of a (demangled or mangled) kernel name: attention, gemm, select..."""
    import re

    if "attn" in name:
        return "attention"
    ids = re.findall(r"([A-Za-z_][A-Za-z0-9_]*?)(?:_kernel)?(?:<[^>]*>)?\(", name)
    ids = [i for i in ids if i not in ("anonymous", "void")]
    if ids:
        return ids[0].split("_kernel")[0]
    m = re.search(r"\d+([a-z_]+?)_kernel", name)  # mangled: ...14combine_kernelI...
    return m.group(1) if m else "kernel"


def summarize_profiles(args):
    """Write profiles/<kernel>_<workload>.md and profiles/traffic_<workload>.json from a
    kernel-trace --stats csv and four --pmc runs (bench FETCH_SIZE / WRITE_SIZE, copy
    FETCH_SIZE / WRITE_SIZE)."""
    import csv

    stats = list(csv.DictReader(open(args.stats)))
    fetch = _pmc_per_kernel(args.fetch, "FETCH_SIZE")
    write = _pmc_per_kernel(args.write, "WRITE_SIZE")
    cfetch = _pmc_per_kernel(args.copy_fetch, "FETCH_SIZE")
    cwrite = _pmc_per_kernel(args.copy_write, "WRITE_SIZE")
    copy_bytes = args.copy_bytes

    def copy_factor(per):
        # largest dispatch of the copy run is the calibration copy
        vals = max((v for vs in per.values() for v in vs), default=0.0)
        return copy_bytes / (vals * 1024.0) if vals else None

    f_fac, w_fac = copy_factor(cfetch), copy_factor(cwrite)
    rows = []
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        fv, wv = fetch.get(name, []), write.get(name, [])
        fb = (sum(fv) / len(fv)) * 1024.0 * f_fac if fv and f_fac else None
        wb = (sum(wv) / len(wv)) * 1024.0 * w_fac if wv and w_fac else None
        rows.append((name, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["Percentage"]), fb, wb))
    sha = kernel_source_sha()
    os.makedirs(PROFILES, exist_ok=True)
    md = [f"# rocprofv3 summary: {args.workload}", "",
          f"kernel sources sha256[:16] = {sha}", "",
          "Commands (run from the repository root on one MI355X; TMPDIR=/tmp):", "```"]
    md += args.commands.split(";;")
    md += ["```", "",
           f"Counter scale: a plain copy of {copy_bytes} bytes reads FETCH_SIZE -> factor "
           f"{f_fac:.4f} and WRITE_SIZE -> factor {w_fac:.4f} bytes per counted byte (KiB x 1024).",
           "", "| kernel | calls | avg us | % time | HBM fetch MB/launch | HBM write MB/launch |",
           "|---|---|---|---|---|---|"]
    for name, calls, us, pct, fb, wb in rows[:16]:
        fbs = f"{fb / 1e6:.2f}" if fb is not None else "-"
        wbs = f"{wb / 1e6:.2f}" if wb is not None else "-"
        md.append(f"| `{name[:90]}` | {calls} | {us:.1f} | {pct:.1f} | {fbs} | {wbs} |")
    dom = rows[0]
    tag = kernel_tag(dom[0])
    out_md = os.path.join(PROFILES, f"{tag}_{args.workload}.md")
    open(out_md, "w").write("\n".join(md) + "\n")
    traffic = {"workload": args.workload, "kernel": dom[0], "source_sha": sha,
               "fetch_bytes_per_launch": dom[4], "write_bytes_per_launch": dom[5],
               "copy_factor_fetch": f_fac, "copy_factor_write": w_fac}
    json.dump(traffic, open(os.path.join(PROFILES, f"traffic_{args.workload}.json"), "w"), indent=1)
    print(out_md)


def ko_weights(wl, ctx):
    """Integer item weights at context ctx (same rounding rule as the library; the library's
    own values are checked against the oracle by the tests)."""
    lat, s = wl.latency, wl.shape
    t = [lat.attn_base + lat.attn_per_token * ctx if i % 2 == 0 else lat.mlp
         for i in range(2 * s.n_layers)]
    delta = sum(t) / (wl.n_budgets - 1)
    return [max(1, int(round(x / delta))) for x in t]


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_prefix(wl, prob, max_layers, seconds):
    """One timed run of the unchanged oracle DP on a bounded prefix of the solve: stopped at
    the first item boundary after ``seconds`` of wall time (or after ``max_layers`` layers).
    A wrapper around the oracle's item function only reads the clock when the next item
    starts, so the timed prefix holds whole items (their forward and their select).  Returns
    (finished items, seconds, FLOP share of the solve those items hold)."""
    from oracle import knapspec_oracle as ko

    s = wl.shape
    shape = ko.DecoderShape(s.n_layers, s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim,
                            s.d_ff, s.rms_eps, s.rope_theta)
    lat = wl.latency
    t = ko.item_latencies(s.n_layers, prob.ctxs[0], lat.attn_base, lat.attn_per_token, lat.mlp)
    w = ko.item_weights(t, wl.n_budgets)
    items = ko.DecoderItems(shape, prob.host_layers, prob.host_kv[0], prob.ctxs[0])
    n_max = 2 * min(max_layers, s.n_layers)

    class _Stop(Exception):
        pass

    t0 = time.perf_counter()
    mark = {"done": 0, "t": 0.0}

    def timed(i, x):
        now = time.perf_counter() - t0
        mark["done"], mark["t"] = i, now  # items 0 .. i-1 are finished
        if i > 0 and now >= seconds:
            raise _Stop
        return items(i, x)

    try:
        ko.knapsack_dp(timed, n_max, w[:n_max], prob.host_x0[0], wl.n_budgets)
        mark["done"], mark["t"] = n_max, time.perf_counter() - t0
    except _Stop:
        pass
    n_items, dt = mark["done"], mark["t"]
    rows, _ = item_rows(list(w), wl.n_budgets)
    d, ff, dh, hq, hkv = s.d_model, s.d_ff, s.head_dim, s.n_q_heads, s.n_kv_heads
    qd, nqkv = hq * dh, (hq + 2 * hkv) * dh

    def item_flops(i):
        R = rows[i]
        if i % 2 == 0:
            return 2.0 * R * (nqkv * d + d * qd) + 4.0 * R * hq * prob.ctxs[0] * dh
        return 2.0 * R * 3 * ff * d
    frac = (sum(item_flops(i) for i in range(n_items)) /
            sum(item_flops(i) for i in range(2 * s.n_layers)))
    return n_items, dt, frac


def cpu_baseline(wl, prob, max_layers, log_fn, seconds=15.0, repeats=3, seconds_1t=8.0):
    """The oracle, untuned, timed on the host cores over a bounded prefix of the same solve
    (see _oracle_prefix), scaled to whole solves by the FLOP share of the finished items.
    ``repeats`` runs with the BLAS pool on every core the process may use give the reported
    value (their median); one more run with a single BLAS thread, capped at ``seconds_1t``,
    is reported beside it."""
    import statistics

    from threadpoolctl import threadpool_info, threadpool_limits

    threads = len(os.sched_getaffinity(0))
    runs = []
    with threadpool_limits(threads):
        for k in range(repeats):
            n_items, dt, frac = _oracle_prefix(wl, prob, max_layers, seconds)
            runs.append((frac / dt, n_items, dt, frac))
            log_fn(f"[cpu] oracle ({threads} threads) run {k}: {n_items} items in {dt:.2f}s = "
                   f"{frac:.3%} of one solve's FLOPs")
    with threadpool_limits(1):
        n1, dt1, frac1 = _oracle_prefix(wl, prob, max_layers, seconds_1t)
    log_fn(f"[cpu] oracle (1 thread): {n1} items in {dt1:.2f}s = {frac1:.3%} of one solve")
    med = statistics.median(r[0] for r in runs)
    blas = sorted({i.get("internal_api", "?") for i in threadpool_info()})
    n_items = [r[1] for r in runs]
    return {"value": med, "unit": "solves/s", "cores": threads, "kind": "oracle",
            "sample": (f"median of {repeats} runs of the first items of one {wl.name} solve "
                       f"({n_items} of {2 * wl.shape.n_layers} items; each stopped at the first "
                       f"item boundary after {seconds:g} s), scaled by their FLOP share"),
            "repeats": [round(r[0], 6) for r in runs],
            "value_1_thread": frac1 / dt1 if dt1 > 0 else None,
            "sample_1_thread": f"first {n1} items in {dt1:.1f}s (FLOP share {frac1:.4f})",
            "cpu_model": cpu_model(), "blas": blas}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b_32k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=1000)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-repeats", type=int, default=3)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--summarize-profiles", action="store_true")
    ap.add_argument("--stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--commands", default="")
    ap.add_argument("--window", type=int, default=1,
                    help="tokens per DP state (r-token window); 1 = the single-token solve")
    ap.add_argument("--beam", type=int, default=1,
                    help="states kept per DP cell (the beam variant); 1 = the one-state DP")
    ap.add_argument("--lm-vocab", type=int, default=0,
                    help="also run the LM-head acceptance estimate with this many rows")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the KnapSpec DP solve runs on a single MI355X "
              "(multi-GPU sharding is a design note, not part of this build); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from workloads import WORKLOADS
    from workloads.device import DeviceProblem

    wl = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    want_cpu = not args.no_cpu_baseline
    t0 = time.time()
    log(f"[bench] generating and uploading {wl.name} inputs ...")
    if args.window != 1 or args.lm_vocab or args.beam != 1:
        want_cpu = False  # the CPU baseline leg covers the single-token solve only
    prob = DeviceProblem(wl, args.seed, keep_host=want_cpu, window=args.window,
                         lm_vocab=args.lm_vocab, max_beam=args.beam)
    flags = prob.ks.KNAPSPEC_ALPHA_LM_HEAD if args.lm_vocab else 0
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s; warmup {args.warmup}")
    # one step = one solve; for a multi-sequence preset one step is its whole re-solve
    # schedule (every sequence re-solved `resolves` times as its context grows)
    multi = prob.n_resolves > 1
    solves_per_step = len(prob.ctxs) * prob.n_resolves

    def step(res):
        if not multi:
            return prob.solve(result=res, flags=flags, beam=args.beam)
        for r in range(prob.n_resolves):
            res = prob.solve(resolve=r, flags=flags, beam=args.beam)
        return res

    res = None
    for _ in range(args.warmup):
        res = step(res)
    torch.cuda.synchronize()

    # timed region: K steps back to back (the headline number)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        res = step(res)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    log(f"[bench] {args.steps} steps ({args.steps * solves_per_step} solves) in {elapsed:.3f}s")

    # roofline region: the same K solves again with every kernel launch bracketed by HIP
    # events on the solve stream (per-kernel-class durations; adds event records per launch)
    prob.model.set_profiling(True)
    torch.cuda.synchronize()
    t_prof = time.perf_counter()
    for _ in range(args.steps):
        res = step(res)
    torch.cuda.synchronize()
    elapsed_prof = time.perf_counter() - t_prof
    ktimes = prob.model.kernel_times()
    prob.model.set_profiling(False)
    log(f"[bench] profiled pass: {args.steps} solves in {elapsed_prof:.3f}s")

    solves_per_s = args.steps * solves_per_step / elapsed
    ms_per_step = 1000.0 * elapsed / args.steps
    # algorithmic work of one step (summed over the schedule's solves)
    cls, tot = None, None
    for r in range(prob.n_resolves):
        ctxs = prob.resolve_ctxs(r) if multi else prob.ctxs
        w_per_seq = [ko_weights(wl, c) for c in ctxs]
        c_r, t_r = algorithmic_work(wl, w_per_seq, ctxs, args.window, args.lm_vocab, args.beam)
        if cls is None:
            cls, tot = c_r, t_r
        else:
            for k in cls:
                for f in ("bytes", "flops", "launches"):
                    cls[k][f] += c_r[k][f]
            for f in ("weight_bytes", "kv_bytes", "state_bytes", "total_bytes", "total_flops"):
                tot[f] += t_r[f]
    achieved_gbs = tot["total_bytes"] * args.steps / elapsed / 1e9

    # dominant kernel class by measured time
    per_class = {}
    for k, (ms, n) in ktimes.items():
        if n:
            per_class[k] = {"total_ms": ms, "launches": n, "avg_us": 1000.0 * ms / n}
    dom = max((k for k in per_class if k in cls), key=lambda k: per_class[k]["total_ms"])
    c = cls[dom]
    avg_s = per_class[dom]["avg_us"] * 1e-6
    bytes_per_launch = c["bytes"] / c["launches"]
    flops_per_launch = c["flops"] / c["launches"]
    ridge = MFMA_PEAK_TFLOPS[wl.shape.dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flops_per_launch / max(1.0, bytes_per_launch) > ridge:
        achieved = flops_per_launch / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2),
                "peak": MFMA_PEAK_TFLOPS[wl.shape.dtype], "unit": "TFLOP/s"}
    else:
        achieved = bytes_per_launch / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None
    tpath = os.path.join(PROFILES, f"traffic_{wl.name}.json")
    if os.path.exists(tpath):
        tr = json.load(open(tpath))
        kname = "attn_mfma" if dom == "attention" else dom
        if (tr.get("source_sha") == kernel_source_sha() and kname in tr.get("kernel", "")
                and tr.get("fetch_bytes_per_launch") is not None):
            roof["traffic"] = int(tr["fetch_bytes_per_launch"] + (tr["write_bytes_per_launch"] or 0))
            roof["traffic_algorithmic"] = int(bytes_per_launch)
    roof["kernel"] = dom
    roof["timer"] = ("average launch duration from HIP events recorded around each launch on "
                     "the solve stream (profiled pass)")
    log("[bench] kernel classes (avg us/launch, share of solve):")
    tot_ms = sum(v["total_ms"] for v in per_class.values())
    for k, v in sorted(per_class.items(), key=lambda kv: -kv[1]["total_ms"]):
        log(f"   {k:14s} {v['avg_us']:9.1f} us x {v['launches'] // args.steps:4d}/solve "
            f"{100 * v['total_ms'] / tot_ms:5.1f}%")

    cpu = None
    if want_cpu:
        try:
            cpu = cpu_baseline(wl, prob, args.cpu_layers, log, args.cpu_seconds,
                               args.cpu_repeats)
        except Exception as e:  # the baseline is reported, never required for the GPU number
            log(f"[cpu] baseline failed: {e!r}")
    headline = (wl.name == "llama3_8b_32k" and args.window == 1 and args.beam == 1
                and not args.lm_vocab)
    variant = "".join([f", window {args.window}" if args.window != 1 else "",
                       f", beam {args.beam}" if args.beam != 1 else "",
                       f", LM head {args.lm_vocab}" if args.lm_vocab else ""])
    line = {
        "metric": METRIC if headline else
                  f"KnapSpec DP solves/sec + achieved HBM GB/s, {wl.name}{variant}",
        "value": round(solves_per_s, 3),
        "unit": "solves/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.shape.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "resolves": prob.n_resolves, "layers": wl.shape.n_layers, "d_model": wl.shape.d_model,
                   "heads_q_kv": [wl.shape.n_q_heads, wl.shape.n_kv_heads],
                   "head_dim": wl.shape.head_dim, "d_ff": wl.shape.d_ff, "ctx": prob.ctxs,
                   "budgets": wl.n_budgets, "gamma": list(wl.gamma), "n_seqs": len(prob.ctxs),
                   "window": args.window, "lm_vocab": args.lm_vocab, "beam": args.beam,
                   "parallelism": "single-gpu"},
        "achieved_hbm_gbs": round(achieved_gbs, 1),
        "hbm_frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": int(tot["total_bytes"]),
        "algorithmic_flops_per_step": float(tot["total_flops"]),
        "solves_per_step": solves_per_step,
        "mfma_frac": round(tot["total_flops"] * args.steps / elapsed / 1e12 /
                           MFMA_PEAK_TFLOPS[wl.shape.dtype], 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernel_us": {k: round(v["avg_us"], 2) for k, v in per_class.items()},
        "kernel_ms_per_solve": round(tot_ms / args.steps, 4),
        "ms_per_step_profiled": round(1000.0 * elapsed_prof / args.steps, 4),
        "best": {"budget": int(res.best_budget[0]), "gamma": int(res.best_gamma[0])},
        "note": ("multi-sequence preset: one step = every sequence re-solved on its schedule; "
                 "value counts single-sequence solves") if multi else None,
    }
    print(json.dumps(line), flush=True)
    prob.close()


if __name__ == "__main__":
    main()

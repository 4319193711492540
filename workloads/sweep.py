"""Context-length sweep, tau ablation and item-latency profiling of the DP on one GPU.

Experiments the KnapSpec pages describe around the DP, run on seeded synthetic inputs:

* Context sweep ("KnapSpec" review, "The reading" and "Load-bearing premise"): the Attention
  item's latency grows linearly with the context length n while the MLP item's is flat, so as
  n grows the DP's budgets buy fewer Attention items; the sweep re-solves the same decoder
  and state at several n and reports, per n, the item weights, the TPT pick, and how many
  Attention and MLP items the picked layer set and the average budget keep.
* Tau ablation ("KnapSpec" review, free parameter tau = 0.5; Figure 4 caption): solve time and
  the number of live DP states per item as the cosine-pruning threshold tau varies.
* Item latency profile: one decode token through an Attention item at several n and through
  an MLP item, timed on the device (knapspec_profile_items), with t_attn(n) = a + b*n fitted
  by least squares (knapspec_fit_latency) -- the measured latency model the weights can use
  instead of the bandwidth stand-in of the presets.
* Beam gap ("KnapSpec" review, "Reading between the lines": an exact or beam-search variant
  shows the greedy rule's headroom): the same problem solved with the one-state DP and with
  beams of k states per cell; per budget, how much higher the best set's cosine is, and how
  the TPT pick and its value change.
* Draft/verify timing (review, "The reading": the draft runs the chosen items, the target
  verifies): the TPT pick (S*, gamma*) run as a masked draft of gamma* tokens and a
  (gamma*+1)-token verification pass (knapspec_draft_verify), against the same draft with
  every item (the target decoding token by token).  Speed only: the synthetic weights make
  acceptance meaningless.

Everything runs through the library (no arithmetic of the method here); this module only
arranges calls and tabulates what the library returns.  Command line:
    python -m workloads.sweep --workload llama3_8b_32k --ctx 1024,4096,16384,32768 --out f.json
"""
from __future__ import annotations

import argparse
import json
import math
import time
from typing import List, Optional, Sequence

import numpy as np

from .configs import WORKLOADS, Workload, scaled


def _mask_bits(masks: np.ndarray, n_items: int) -> np.ndarray:
    """[B][mw] uint64 -> [B][n_items] bool (bit i of word i // 64 = item i executed)."""
    words = masks.astype(np.uint64)
    bits = np.zeros((words.shape[0], n_items), dtype=bool)
    for i in range(n_items):
        bits[:, i] = ((words[:, i // 64] >> np.uint64(i % 64)) & np.uint64(1)) == 1
    return bits


def layer_set_stats(res, q: int, n_items: int) -> dict:
    """Attention / MLP items kept by the TPT pick and on average over valid budgets."""
    bits = _mask_bits(res.masks[q], n_items)
    valid = res.valid[q].astype(bool)
    attn = bits[:, 0::2].sum(axis=1)
    mlp = bits[:, 1::2].sum(axis=1)
    L = n_items // 2
    out = {"valid_budgets": int(valid.sum())}
    b = int(res.best_budget[q])
    if b >= 0:
        out.update(pick_budget=b, pick_gamma=int(res.best_gamma[q]),
                   pick_attn_kept=int(attn[b]), pick_mlp_kept=int(mlp[b]),
                   pick_cos=float(res.cos[q][b]))
    if valid.any():
        out.update(mean_attn_kept_frac=float(attn[valid].mean() / L),
                   mean_mlp_kept_frac=float(mlp[valid].mean() / L))
    return out


def context_sweep(prob, ctx_list: Sequence[int], n_budgets: Optional[int] = None,
                  gamma=None) -> List[dict]:
    """Re-solve the problem at each context length (same weights, caches, x0)."""
    wl = prob.wl
    n_items = 2 * wl.shape.n_layers
    rows = []
    for n in ctx_list:
        res = prob.solve(n_budgets=n_budgets, gamma=gamma, ctxs=[int(n)])
        w = res.item_weight[0]
        row = {"ctx": int(n), "w_attn": int(w[0]), "w_mlp": int(w[1]),
               "sum_w": int(w.sum())}
        row.update(layer_set_stats(res, 0, n_items))
        rows.append(row)
    return rows


def tau_ablation(prob, taus: Sequence[float], reps: int = 5, n_budgets: Optional[int] = None,
                 gamma=None) -> List[dict]:
    """Solve time (median of reps, host clock around the synchronous solve) and live states
    per item (cells whose decision is not 'invalid') for each tau.  With pruning on, the solve
    drops pruned budgets' rows on the device; ``solve_ms_kept_rows`` times the same solve with
    the rows planned from reachability kept (KNAPSPEC_KEEP_PRUNED_ROWS)."""
    import torch

    wl = prob.wl
    n_items = 2 * wl.shape.n_layers
    keep = prob.ks.KNAPSPEC_KEEP_PRUNED_ROWS

    def timed(tau, flags):
        for _ in range(2):  # untimed: the first solves of a configuration capture its graph
            prob.solve(n_budgets=n_budgets, gamma=gamma, tau=tau, flags=flags)
        times = []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            prob.solve(n_budgets=n_budgets, gamma=gamma, tau=tau, flags=flags)
            times.append(time.perf_counter() - t0)
        return 1e3 * float(np.median(times))

    rows = []
    for tau in taus:
        res = prob.solve(n_budgets=n_budgets, gamma=gamma, tau=tau, flags=1)  # decisions
        dec = res.decisions[0]
        live = (dec != 255).sum(axis=1)
        row = {"tau": None if math.isinf(tau) else float(tau),
               "solve_ms": timed(tau, 0), "solve_ms_kept_rows": timed(tau, keep),
               "live_states_mean": float(live.mean()), "live_states_last": int(live[-1])}
        row.update(layer_set_stats(res, 0, n_items))
        rows.append(row)
    return rows


def beam_gap(prob, beams: Sequence[int], reps: int = 3, band: Optional[float] = None) -> List[dict]:
    """Per beam width: solve time (median host time of reps) and, against beam 1, how many
    valid budgets end with a set whose cosine is higher by more than ``band`` (default: the
    parity band of the dtype, 2e-3 bf16 / 1e-5 float32 -- smaller differences are rounding
    of differently batched rows), the largest and mean cosine gain, and the TPT pick."""
    if band is None:
        band = 2e-3 if prob.wl.shape.dtype == "bf16" else 1e-5
    import torch

    rows = []
    base = None
    for k in beams:
        res = prob.solve(beam=int(k))
        for _ in range(2):  # untimed: the first solves of a configuration capture its graph
            prob.solve(beam=int(k))
        times = []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            prob.solve(beam=int(k))
            times.append(time.perf_counter() - t0)
        valid = res.valid[0].astype(bool)
        cos = res.cos[0].astype(np.float64)
        row = {"beam": int(k), "solve_ms": 1e3 * float(np.median(times)),
               "valid_budgets": int(valid.sum()), "pick_budget": int(res.best_budget[0]),
               "pick_gamma": int(res.best_gamma[0]), "best_tpt": float(res.best_tpt[0])}
        if base is None:
            base = cos
        else:
            gain = np.where(valid, cos - base, 0.0)
            row.update(band=band, better_budgets=int(np.sum(gain > band)),
                       max_cos_gain=float(gain.max()), mean_cos_gain=float(gain[valid].mean()),
                       p90_cos_gain=float(np.percentile(gain[valid], 90)))
        rows.append(row)
    return rows


def draft_verify_timing(prob, reps: int = 3) -> dict:
    """Device time of the TPT pick's masked draft and of its verification, and of a draft with
    every item executed, at the preset context (median of reps after one warm-up call).
    The caches must hold ctx + gamma* + 1 positions; positions ctx .. ctx+gamma* are written."""
    wl = prob.wl
    n_items = 2 * wl.shape.n_layers
    res = prob.solve()
    b, g = int(res.best_budget[0]), int(res.best_gamma[0])
    g = max(1, min(g, prob.ks.KNAPSPEC_WINDOW_MAX - 1))
    mw = (n_items + 63) // 64
    full = np.zeros(mw, dtype=np.uint64)
    for i in range(n_items):
        full[i // 64] |= np.uint64(1) << np.uint64(i % 64)
    out = {"pick_budget": b, "gamma": g,
           "pick_items": int(_mask_bits(res.masks[0][b:b + 1], n_items).sum()) if b >= 0 else 0,
           "t_draft_model": float(res.t_draft[0][b]) if b >= 0 else None}
    seq = prob.seq_args()[0]
    for name, mask in (("pick", res.masks[0][b] if b >= 0 else full), ("full", full)):
        prob.model.draft_verify(seq, mask, g)  # warm-up
        runs = [prob.model.draft_verify(seq, mask, g) for _ in range(reps)]
        out[f"{name}_draft_us"] = float(np.median([r["draft_us"] for r in runs]))
        out[f"{name}_verify_us"] = float(np.median([r["verify_us"] for r in runs]))
        out[f"{name}_draft_us_per_token"] = out[f"{name}_draft_us"] / g
    return out


def latency_profile(prob, ctx_list: Sequence[int], reps: int = 8) -> dict:
    """Measured item latencies and the fitted linear attention model (microseconds)."""
    seq = prob.seq_args([max(ctx_list)])[0]
    attn, mlp = prob.model.profile_items(seq, list(ctx_list), reps=reps)
    a, b, r2 = prob.ks.fit_latency(list(ctx_list), attn)
    return {"ctx": [int(n) for n in ctx_list], "attn_us": [float(x) for x in attn],
            "mlp_us": float(mlp), "fit_attn_base_us": a, "fit_attn_per_token_us": b,
            "fit_r2": r2}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", default="llama3_8b_32k")
    ap.add_argument("--layers", type=int, default=0, help="keep only the first L layers")
    ap.add_argument("--ctx", default="1024,2048,4096,8192,16384,32768")
    ap.add_argument("--taus", default="-inf,0.0,0.3,0.5,0.7,0.9")
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--beams", default="", help="beam widths for the beam-gap table, e.g. 1,2,4,8")
    ap.add_argument("--draft-verify", type=int, default=0, metavar="VOCAB",
                    help="time the pick's masked draft + verification with an LM head of VOCAB rows")
    ap.add_argument("--profiled", action="store_true",
                    help="also solve the sweep with the measured (fitted) latency model")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--out", default="")
    ap.add_argument("--solves", type=int, default=0, metavar="N",
                    help="only run N solves at each tau of --taus (e.g. under a kernel tracer)")
    ap.add_argument("--kept-rows", action="store_true",
                    help="with --solves: keep the pruned budgets' rows (KNAPSPEC_KEEP_PRUNED_ROWS)")
    ap.add_argument("--batch", action="store_true",
                    help="with --solves: solve all of the preset's sequences together at their "
                         "own contexts (e.g. the 16-sequence preset) instead of one at --ctx")
    args = ap.parse_args(argv)

    from .device import DeviceProblem

    wl: Workload = WORKLOADS[args.workload]
    if args.layers:
        wl = scaled(wl, n_layers=args.layers)
    ctx_list = [int(x) for x in args.ctx.split(",")]
    taus = [float(x) for x in args.taus.split(",")]
    cap = max(max(ctx_list), wl.ctx) + 16  # room for a draft/verify block past the context
    beams = [int(x) for x in args.beams.split(",")] if args.beams else []
    if args.solves and args.batch:
        prob = DeviceProblem(wl, args.seed)
    else:
        prob = DeviceProblem(wl, args.seed, ctxs=[wl.ctx], caps=[cap],
                             max_beam=max(beams) if beams else 1, lm_vocab=args.draft_verify)
    if args.solves:
        import torch

        flags = prob.ks.KNAPSPEC_KEEP_PRUNED_ROWS if args.kept_rows else 0
        for tau in taus:
            for k in range(args.solves):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                res = prob.solve(tau=tau, flags=flags)
                print(f"tau {tau} solve {k}: {1e3 * (time.perf_counter() - t0):.3f} ms, "
                      f"valid budgets {int(res.valid.sum())} over {len(prob.ctxs)} sequences",
                      flush=True)
        prob.close()
        return
    out = {"workload": wl.name, "layers": wl.shape.n_layers, "n_budgets": wl.n_budgets,
           "latency_model": "bandwidth-bound stand-in (8 TB/s)",
           "sweep": context_sweep(prob, ctx_list)}
    print(json.dumps({"sweep": out["sweep"]}), flush=True)
    out["tau_ablation"] = tau_ablation(prob, taus, reps=args.reps)
    print(json.dumps({"tau_ablation": out["tau_ablation"]}), flush=True)
    if beams:
        out["beam_gap"] = beam_gap(prob, beams, reps=args.reps)
        print(json.dumps({"beam_gap": out["beam_gap"]}), flush=True)
    if args.draft_verify:
        out["draft_verify"] = draft_verify_timing(prob, reps=args.reps)
        print(json.dumps({"draft_verify": out["draft_verify"]}), flush=True)
    if len(set(ctx_list)) < 2:  # a line fit needs two context lengths
        prob.close()
        if args.out:
            with open(args.out, "w") as f:
                json.dump(out, f, indent=1)
        return
    prof = latency_profile(prob, ctx_list, reps=max(args.reps, 8))
    out["latency_profile"] = prof
    print(json.dumps({"latency_profile": prof}), flush=True)
    if args.profiled:
        prob.model.set_latency(prof["fit_attn_base_us"], prof["fit_attn_per_token_us"],
                               prof["mlp_us"], 0.0)
        out["sweep_profiled_latency"] = context_sweep(prob, ctx_list)
        print(json.dumps({"sweep_profiled_latency": out["sweep_profiled_latency"]}), flush=True)
    prob.close()
    if args.out:
        with open(args.out, "w") as f:
            json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()

"""Item latency profiling, the context sweep and the tau ablation (workloads.sweep) on the GPU.

* knapspec_profile_items: positive latencies, Attention's growing with the context length,
  a line fit with positive slope, and no effect on the results of solves around it.
* Context sweep: every swept context's solve is checked against the oracle (rules P1-P4), and
  the tabulated layer-set statistics are recomputed from the returned masks.
* Tau ablation: live states never increase with tau, and every ablated solve passes parity.
"""
import math

import numpy as np
import pytest

from oracle import knapspec_oracle as ko
from tests.helpers import decoder_shape
from tests.parity import compare
from workloads import WORKLOADS, scaled

pytestmark = pytest.mark.gpu

BETA = {"f32": 1e-5, "bf16": 2e-3}


def _same(a, b):
    for f in ("masks", "valid", "best_budget", "best_gamma", "item_weight"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert np.array_equal(a.cos, b.cos, equal_nan=True)


def _oracle_check(prob, res, wl, ctx, tau=-math.inf):
    lat = {"attn_base": wl.latency.attn_base, "attn_per_token": wl.latency.attn_per_token,
           "mlp": wl.latency.mlp, "fixed": wl.latency.fixed}
    items = ko.DecoderItems(decoder_shape(wl), prob.host_layers, prob.host_kv[0], ctx,
                            cache_widened=True)
    orc = ko.solve(decoder_shape(wl), None, None, prob.host_x0[0], ctx, lat, wl.n_budgets,
                   wl.gamma, tau=tau, apply_item=items)
    rep = compare(orc, res, 0, BETA[wl.shape.dtype], items, prob.host_x0[0], wl.gamma,
                  2 * wl.shape.n_layers)
    print(f"  ctx={ctx} tau={tau}: {rep.line()}", flush=True)
    assert rep.mismatched_clean == 0
    assert rep.p2_max_err <= BETA[wl.shape.dtype]
    assert rep.p3_bad == 0
    assert rep.p4_ok
    return orc


def test_profile_items_latency_and_fit():
    from workloads.device import DeviceProblem

    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=4, name="profile_t")
    ctxs = [0, 1024, 4096, 8192, 16384]
    print(f"\n[case] profile_items {wl.name} ctxs={ctxs}", flush=True)
    prob = DeviceProblem(wl, 0, ctxs=[wl.ctx], caps=[max(ctxs)])
    before = prob.solve(flags=3)
    seq = prob.seq_args([max(ctxs)])[0]
    attn, mlp = prob.model.profile_items(seq, ctxs, reps=8)
    print(f"  attn_us={np.round(attn, 2).tolist()} mlp_us={mlp:.2f}", flush=True)
    assert np.all(attn > 0) and mlp > 0
    assert attn[-1] > attn[0]  # reading 16K cached positions costs more than none
    a, b, r2 = prob.ks.fit_latency(ctxs, attn)
    print(f"  fit: a={a:.3f} us, b={b:.3e} us/token, r2={r2:.3f}", flush=True)
    assert b > 0 and r2 > 0.5
    after = prob.solve(flags=3)
    _same(before, after)
    prob.close()


def test_context_sweep_parity():
    from workloads.device import DeviceProblem
    from workloads.sweep import context_sweep, layer_set_stats

    wl = WORKLOADS["tiny"]
    ctxs = [0, 64, 256, 512]
    print(f"\n[case] context sweep {wl.name} ctxs={ctxs}", flush=True)
    prob = DeviceProblem(wl, 0, ctxs=[wl.ctx], caps=[max(ctxs)], keep_host=True)
    rows = context_sweep(prob, ctxs)
    for row in rows:
        print(f"  {row}", flush=True)
    n_items = 2 * wl.shape.n_layers
    for n, row in zip(ctxs, rows):
        res = prob.solve(ctxs=[n], flags=3)
        orc = _oracle_check(prob, res, wl, n)
        assert row == {**{"ctx": n, "w_attn": int(orc.w[0]), "w_mlp": int(orc.w[1]),
                          "sum_w": int(np.sum(orc.w))}, **layer_set_stats(res, 0, n_items)}
    # the Attention item's weight never falls as the context grows
    w_attn = [r["w_attn"] for r in rows]
    assert w_attn == sorted(w_attn)
    prob.close()


def test_tau_ablation_parity():
    from workloads.device import DeviceProblem
    from workloads.sweep import tau_ablation

    wl = scaled(WORKLOADS["tiny"], n_layers=5, n_kv_heads=2, name="tau_t")
    taus = [-math.inf, 0.0, 0.5, 0.9]
    print(f"\n[case] tau ablation {wl.name} taus={taus}", flush=True)
    prob = DeviceProblem(wl, 1, ctxs=[130], keep_host=True)
    rows = tau_ablation(prob, taus, reps=2)
    for row in rows:
        print(f"  {row}", flush=True)
    live = [r["live_states_mean"] for r in rows]
    assert all(x >= y for x, y in zip(live, live[1:]))
    for tau in taus:
        res = prob.solve(tau=tau, flags=3)
        _oracle_check(prob, res, wl, 130, tau=tau)
    prob.close()

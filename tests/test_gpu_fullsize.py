"""Full-size presets on the GPU, in the launch configuration bench.py times.

Llama-3-8B 32K (the headline) and the 16-sequence re-solve schedule are compared with the
oracle's WHOLE DP (tests/parity.py: P1 on every cell, P2 on every valid budget's mask, P3 on
the valid sets, P4 on the (b, gamma) pick), the oracle's forward of the GPU's masks riding
along the DP's item calls (helpers.LockstepSubsets).  Every case also checks properties that
hold at any size: item weights equal the oracle's; valid budgets are exactly the reachable
weight sums; every valid mask's weights sum to its budget; the per-cell decisions walk back to
the returned masks; t_draft is the sum of the executed items' latencies; the (b, gamma) pick
is the TPT argmax of the returned cosines.  The bench's variant lines at full size (r = 5
windows with the LM-head estimate, and beam 4) are checked on those properties, P2 on sampled
masks and, for the window, the greedy tokens of the sampled budgets and of the full model
against the oracle's (tokens inside the logit band excused).
"""
import math
import time

import numpy as np
import pytest

from oracle import knapspec_oracle as ko
from tests.helpers import decoder_shape
from workloads import WORKLOADS

pytestmark = pytest.mark.gpu

BETA = {"f32": 1e-5, "bf16": 2e-3}


def reachable(w, B):
    r = np.zeros(B, dtype=bool)
    r[0] = True
    for wi in w:
        nr = r.copy()
        nr[wi:] |= r[: B - wi]
        r = nr
    return r


def check_structure(res, q, t, B, gamma, n_items, t_target, decisions=True, alpha=None):
    w = res.item_weight[q].astype(np.int64)
    valid = res.valid[q].astype(bool)
    assert np.array_equal(valid, reachable(w, B))
    bits = ko.unpack_masks(res.masks[q], n_items)
    for b in range(B):
        if valid[b]:
            assert int(np.sum(w[bits[b]])) == b, b
            assert res.t_draft[q][b] == pytest.approx(float(np.sum(t[bits[b]])), rel=1e-12)
        else:
            assert not bits[b].any()
    dec = res.decisions[q] if decisions else None
    for b0 in (np.nonzero(valid)[0] if decisions else []):
        b, got = int(b0), np.zeros(n_items, dtype=bool)
        for i in range(n_items - 1, -1, -1):
            assert dec[i][b] in (0, 1)
            if dec[i][b] == 1:
                got[i] = True
                b -= int(w[i])
        assert b == 0 and np.array_equal(got, bits[b0])
    c = res.cos[q]
    assert np.all(c[valid] <= 1.0 + 1e-6) and np.all(np.isnan(c[~valid]))
    if alpha is None:
        alpha = np.clip(np.nan_to_num(c.astype(np.float64), nan=0.0), 0.0, 1.0)
    pick = ko.tpt_select(alpha, res.t_draft[q], valid, t_target, gamma[0], gamma[1])
    assert (pick[0], pick[1]) == (int(res.best_budget[q]), int(res.best_gamma[q]))


def full_parity(layers, prob, res, q, wl, ctx, x0, label="", tau=-math.inf, skip_cap=-1):
    """The oracle's whole solve for sequence q against the GPU's (P1-P4 on every cell), with
    the same tau / skip-cap pruning."""
    from tests.helpers import LockstepSubsets
    from tests.parity import compare

    s = wl.shape
    n_items = 2 * s.n_layers
    lat = {"attn_base": wl.latency.attn_base, "attn_per_token": wl.latency.attn_per_token,
           "mlp": wl.latency.mlp, "fixed": wl.latency.fixed}
    items = ko.DecoderItems(decoder_shape(wl), layers, prob.host_kv[q], ctx)
    valid = np.nonzero(res.valid[q])[0]
    bits = ko.unpack_masks(res.masks[q], n_items)[valid]
    lock = LockstepSubsets(items, x0, bits)
    t0 = time.time()
    orc = ko.solve(decoder_shape(wl), None, None, x0, ctx, lat, wl.n_budgets, wl.gamma,
                   tau=tau, skip_cap=skip_cap, apply_item=lock)
    p2 = np.full(wl.n_budgets, np.nan)
    p2[valid] = lock.cos(orc.dp.ref)
    rep = compare(orc, res, q, BETA[s.dtype], None, x0, wl.gamma, n_items, p2_cos=p2)
    print(f"  {label}seq {q} ctx {ctx}: oracle DP + P2 in {time.time() - t0:.1f}s; "
          f"{rep.line()}; pick gpu ({int(res.best_budget[q])}, {int(res.best_gamma[q])}) "
          f"oracle ({orc.best_budget}, {orc.best_gamma})", flush=True)
    assert rep.mismatched_clean == 0
    assert rep.p2_max_err <= BETA[s.dtype]
    assert rep.p3_bad == 0
    assert rep.p4_ok
    return orc, rep


@pytest.mark.timeout(900)
def test_llama3_8b_32k_full():
    from tests.helpers import WidenedLayers
    from workloads.device import DeviceProblem

    wl = WORKLOADS["llama3_8b_32k"]
    print(f"\n[case] {wl.name} full size, whole-DP parity", flush=True)
    prob = DeviceProblem(wl, 0, keep_host=True)
    res = prob.solve(flags=3)
    res2 = prob.solve(flags=3)
    assert np.array_equal(res.masks, res2.masks) and np.array_equal(res.decisions, res2.decisions)
    s, lat = wl.shape, wl.latency
    t = ko.item_latencies(s.n_layers, prob.ctxs[0], lat.attn_base, lat.attn_per_token, lat.mlp)
    check_structure(res, 0, t, wl.n_budgets, wl.gamma, 2 * s.n_layers, float(np.sum(t)))
    full_parity(WidenedLayers(prob.host_layers), prob, res, 0, wl, prob.ctxs[0],
                prob.host_x0[0])
    prob.close()


@pytest.mark.timeout(1100)
def test_llama3_8b_x16_resolve_schedule():
    """16 sequences, contexts lognormal in [2K, 32K], re-solved every 256 tokens (8 times),
    all sequences batched into each solve.  Every sequence of every re-solve is checked for
    the structural properties; every sequence at the first and the last re-solve against
    the oracle's whole DP."""
    from tests.helpers import WidenedLayers
    from workloads.device import DeviceProblem

    wl = WORKLOADS["llama3_8b_x16"]
    print(f"\n[case] {wl.name}", flush=True)
    prob = DeviceProblem(wl, 0, keep_host=True)
    print(f"  contexts {prob.ctxs}", flush=True)
    layers = WidenedLayers(prob.host_layers, keep_all=True)
    s = wl.shape
    n_items = 2 * s.n_layers
    lat = wl.latency
    for r in range(wl.resolves):
        res = prob.solve(flags=3, resolve=r)
        ctxs = prob.resolve_ctxs(r)
        for q in range(len(ctxs)):
            t = ko.item_latencies(s.n_layers, ctxs[q], lat.attn_base, lat.attn_per_token, lat.mlp)
            w = ko.item_weights(t, wl.n_budgets)
            assert np.array_equal(res.item_weight[q], w.astype(np.int32))
            check_structure(res, q, t, wl.n_budgets, wl.gamma, n_items, float(np.sum(t)))
        print(f"  resolve {r}: picks {[(int(b), int(g)) for b, g in zip(res.best_budget, res.best_gamma)]}",
              flush=True)
        if r in (0, wl.resolves - 1):
            for q in range(len(ctxs)):
                full_parity(layers, prob, res, q, wl, ctxs[q], prob.resolve_x0[q][r],
                            label=f"resolve {r} ")
    prob.close()


def sample_budgets(res, q, n_sample, rng):
    valid = np.nonzero(res.valid[q])[0]
    picks = set(rng.choice(valid, size=min(n_sample, len(valid)), replace=False).tolist())
    picks |= {int(valid[0]), int(valid[-1])}
    if res.best_budget[q] >= 0:
        picks.add(int(res.best_budget[q]))
    return sorted(picks)


@pytest.mark.timeout(900)
def test_llama3_8b_32k_full_window5_lm_head():
    from tests.parity import forward_states
    from workloads.device import DeviceProblem

    wl = WORKLOADS["llama3_8b_32k"]
    s = wl.shape
    r, vocab, band = 5, 32768, 0.05
    print(f"\n[case] {wl.name} full size, window r={r}, LM head {vocab}", flush=True)
    prob = DeviceProblem(wl, 0, keep_host=True, window=r, lm_vocab=vocab)
    res = prob.solve(flags=3 | prob.ks.KNAPSPEC_ALPHA_LM_HEAD)
    n_items, ctx, x0 = 2 * s.n_layers, prob.ctxs[0], prob.host_x0[0]
    lat = wl.latency
    t = ko.item_latencies(s.n_layers, ctx, lat.attn_base, lat.attn_per_token, lat.mlp)
    w = ko.item_weights(t, wl.n_budgets)
    assert np.array_equal(res.item_weight[0], w.astype(np.int32))
    check_structure(res, 0, t, wl.n_budgets, wl.gamma, n_items, float(np.sum(t)),
                    alpha=res.alpha[0].astype(np.float64))
    items = ko.DecoderItems(decoder_shape(wl), prob.host_layers, prob.host_kv[0], ctx)
    picks = sample_budgets(res, 0, 5, np.random.default_rng(2))
    bits = ko.unpack_masks(res.masks[0], n_items)[picks]
    t0 = time.time()
    st, ref = forward_states(items, n_items, x0, bits)
    cos = np.array([ko.cos_rows(st[k][None], ref)[0] for k in range(len(picks))])
    err = np.abs(cos - res.cos[0][picks].astype(np.float64))
    print(f"  P2 on budgets {picks}: max err {err.max():.2e} ({time.time() - t0:.1f}s)", flush=True)
    assert err.max() <= BETA[s.dtype]
    # greedy tokens of the sampled budgets and of the full model
    tok_g = res.tokens(0)
    tok_o, mar_o = ko.greedy_tokens(st, prob.host_lm, s.rms_eps)
    tref, mref = ko.greedy_tokens(np.asarray(ref).reshape(r, -1), prob.host_lm, s.rms_eps)
    B = wl.n_budgets
    clean_ref = mref >= band
    assert np.all((tok_g[B] == tref) | ~clean_ref)
    mism = excused = 0
    for k, b in enumerate(picks):
        clean = (mar_o[k] >= band) & clean_ref
        excused += int(np.sum(~clean))
        mism += int(np.sum((tok_g[b] != tok_o[k]) & clean))
        assert abs(float(res.alpha[0][b]) - float(np.sum(tok_g[b] == tok_g[B])) / r) <= 1e-6
    print(f"  tokens: {len(picks) * r} compared, {excused} excused, {mism} mismatched", flush=True)
    assert mism == 0
    prob.close()


@pytest.mark.timeout(900)
def test_llama3_8b_32k_full_beam4():
    from workloads.device import DeviceProblem

    wl = WORKLOADS["llama3_8b_32k"]
    s = wl.shape
    print(f"\n[case] {wl.name} full size, beam 4", flush=True)
    prob = DeviceProblem(wl, 0, keep_host=True, max_beam=4)
    res = prob.solve(beam=4)
    n_items, ctx, x0 = 2 * s.n_layers, prob.ctxs[0], prob.host_x0[0]
    lat = wl.latency
    t = ko.item_latencies(s.n_layers, ctx, lat.attn_base, lat.attn_per_token, lat.mlp)
    w = ko.item_weights(t, wl.n_budgets)
    assert np.array_equal(res.item_weight[0], w.astype(np.int32))
    check_structure(res, 0, t, wl.n_budgets, wl.gamma, n_items, float(np.sum(t)),
                    decisions=False)
    items = ko.DecoderItems(decoder_shape(wl), prob.host_layers, prob.host_kv[0], ctx)
    picks = sample_budgets(res, 0, 6, np.random.default_rng(3))
    bits = ko.unpack_masks(res.masks[0], n_items)[picks]
    t0 = time.time()
    ev = ko.eval_subsets(items, n_items, x0, bits)
    err = np.abs(ev - res.cos[0][picks].astype(np.float64))
    print(f"  P2 on budgets {picks}: max err {err.max():.2e} ({time.time() - t0:.1f}s)", flush=True)
    assert err.max() <= BETA[s.dtype]
    prob.close()

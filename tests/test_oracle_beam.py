"""Pins for the beam variant of the DP (top-k states per cell).

* beam 1 reproduces the one-state DP exactly (sets, cosines, validity, states);
* a beam as wide as the largest number of subsets of one weight keeps every subset, so each
  budget's best set is the best subset of that weight found by enumeration (brute force);
* every kept set has the weight of its budget and re-running it gives its cosine; slots are
  ordered by cosine.
"""
import numpy as np
import pytest

from oracle import knapspec_oracle as ko
from tests.helpers import decoder_shape
from workloads import WORKLOADS, scaled, synth


def _problem(n_layers=4, r=1, ctx=40):
    wl = scaled(WORKLOADS["tiny"], n_layers=n_layers, name="beam_t")
    layers = [synth.layer_weights(wl, l, 0) for l in range(n_layers)]
    kv = [synth.kv_cache(wl, l, 0, 64, 0) for l in range(n_layers)]
    x0 = synth.x0(wl, 0, 0, 0) if r == 1 else synth.x0_window(wl, r, 0, 0, 0)
    items = ko.DecoderItems(decoder_shape(wl), layers, kv, ctx, cache_widened=True)
    t = ko.item_latencies(n_layers, ctx, 1.0, 0.01, 2.0)
    return wl, items, x0, ko.item_weights(t, 14)


@pytest.mark.parametrize("tau", [-np.inf, 0.3])
def test_beam_one_is_the_greedy_dp(tau):
    wl, items, x0, w = _problem()
    n = 2 * wl.shape.n_layers
    g = ko.knapsack_dp(items, n, w, x0, 14, tau=tau)
    b = ko.knapsack_dp_beam(items, n, w, x0, 14, 1, tau=tau).best()
    assert np.array_equal(g.bits, b.bits)
    assert np.array_equal(g.valid, b.valid)
    # the same float64 cosines up to the summation order of the batched dot products
    assert np.allclose(g.cos, b.cos, rtol=0, atol=1e-12, equal_nan=True)
    assert np.array_equal(g.states, b.states)


@pytest.mark.parametrize("r", [1, 2])
def test_wide_beam_is_exhaustive_enumeration(r):
    wl, items, x0, w = _problem(r=r)
    n = 2 * wl.shape.n_layers
    ids, cos_all = ko.brute_force(items, n, x0)
    weight = np.array([sum(int(w[i]) for i in range(n) if (s >> i) & 1) for s in ids])
    widest = int(max(np.sum(weight == b) for b in range(14)))
    res = ko.knapsack_dp_beam(items, n, w, x0, 14, widest)
    greedy = ko.knapsack_dp(items, n, w, x0, 14)
    gaps = []
    for b in range(14):
        sel = weight == b
        assert res.valid[b, 0] == bool(sel.any())
        if not sel.any():
            continue
        assert res.cos[b, 0] == pytest.approx(float(cos_all[sel].max()), abs=1e-6)
        # every subset of weight b is kept
        assert int(res.valid[b].sum()) == int(sel.sum())
        gaps.append(float(cos_all[sel].max()) - greedy.cos[b])
    assert min(gaps) >= -1e-6
    print(f"\n[beam exhaustive r={r}] beam={widest} budgets={len(gaps)} "
          f"greedy optimal={sum(g < 1e-6 for g in gaps)} max_gap={max(gaps):.3e}")


def test_beam_slots_are_consistent():
    wl, items, x0, w = _problem()
    n = 2 * wl.shape.n_layers
    res = ko.knapsack_dp_beam(items, n, w, x0, 14, 3)
    for b in range(14):
        vs = np.nonzero(res.valid[b])[0]
        assert list(vs) == list(range(len(vs)))             # kept slots are a prefix
        c = res.cos[b, vs]
        assert np.all(np.diff(c) <= 0)                      # ordered by cosine
        for j in vs:
            assert int(np.sum(w[res.bits[b, j]])) == b
            cj = ko.eval_subsets(items, n, x0, res.bits[b, j][None])[0]
            assert cj == pytest.approx(res.cos[b, j], abs=1e-6)
        # kept sets are distinct
        assert len({res.bits[b, j].tobytes() for j in vs}) == len(vs)

"""Pins for the oracle's whole-solve composition (latencies -> weights -> DP -> t_draft /
t_target -> acceptance proxy -> TPT grid) and for the acceptance proxy clamp(cos, 0, 1).

The expected values are derived by hand in tests/golden/solve_fixed_hand_values.json: a
four-item decoder whose items add mutually orthogonal vectors, so the cosine of every set has
a closed form and the DP's per-budget sets are the exact knapsack optimum, with a non-zero
per-pass latency `fixed` that moves the TPT pick into the interior of the (b, gamma) grid.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import knapspec_oracle as ko

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "solve_fixed_hand_values.json")


def _additive_items(norm_sq, d=8):
    U = np.zeros((len(norm_sq), d), dtype=np.float32)
    for i, v in enumerate(norm_sq):
        U[i, i + 1] = math.sqrt(v)

    def apply_item(i, X):
        return (X + U[i]).astype(np.float32)
    return apply_item


def _solve(case, fixed=None):
    lat = dict(case["latency"])
    if fixed is not None:
        lat["fixed"] = fixed
    shape = ko.DecoderShape(2, 8, 1, 1, 8, 8)
    x0 = np.zeros(8, dtype=np.float32)
    x0[0] = 1.0
    return ko.solve(shape, None, None, x0, case["ctx"], lat, case["n_budgets"],
                    case["gamma"], apply_item=_additive_items(case["item_norm_sq"]))


def test_solve_with_fixed_latency_hand_values():
    case = json.load(open(GOLDEN))
    o = _solve(case)
    assert o.w.tolist() == case["weights"]
    assert o.t.tolist() == [1.0, 2.0, 1.0, 2.0]
    assert o.t_target == case["t_target"]
    assert o.t_draft.tolist() == case["t_draft"]
    for b, items in enumerate(case["masks"]):
        assert np.nonzero(o.dp.bits[b])[0].tolist() == items, b
    assert o.dp.valid.all()
    assert np.allclose(o.dp.cos, case["cos"], rtol=0, atol=1e-7)
    assert (o.best_budget, o.best_gamma) == (case["best_budget"], case["best_gamma"])
    assert o.best_tpt == pytest.approx(case["best_tpt"], rel=1e-6)
    # the pick is interior in both budget and gamma
    assert 0 < o.best_budget < case["n_budgets"] - 1
    assert case["gamma"][0] < o.best_gamma < case["gamma"][1]


def test_fixed_latency_moves_the_pick():
    case = json.load(open(GOLDEN))
    o = _solve(case, fixed=0.0)
    assert o.t_target == 6.0 and o.t_draft[0] == 0.0
    assert [o.best_budget, o.best_gamma] == case["best_with_fixed_zero"]


def test_alpha_from_cos_clamps_and_maps_nan_to_zero():
    got = ko.alpha_from_cos(np.array([-0.3, 0.4, 1.2, np.nan, -np.inf, np.inf, 0.0, 1.0],
                                     dtype=np.float32))
    want = [0.0, 0.4, 1.0, 0.0, 0.0, 1.0, 0.0, 1.0]
    assert got.dtype == np.float64
    assert np.allclose(got, want, rtol=0, atol=1e-7)
    # float32 inputs are widened, not rounded again
    assert ko.alpha_from_cos(np.array([0.4], dtype=np.float32))[0] == float(np.float32(0.4))


def test_solve_uses_alpha_from_cos_for_the_grid():
    case = json.load(open(GOLDEN))
    o = _solve(case)
    assert np.array_equal(o.alpha, np.clip(o.dp.cos, 0.0, 1.0))

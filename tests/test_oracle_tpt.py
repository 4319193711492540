"""Pins for the oracle's Tokens-per-Time objective and grid search (KnapSpec Eq. 4)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import knapspec_oracle as ko

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tpt_hand_values.json")


def test_hand_derived_values():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        v = ko.tpt_value(c["alpha"], c["gamma"], c["t_draft"], c["t_target"])
        assert v == pytest.approx(c["tpt"], rel=1e-14, abs=0), c


@pytest.mark.parametrize("alpha", [0.0, 1e-9, 0.1, 0.37, 0.5, 0.8, 0.99, 0.999999, 1 - 1e-7, 1.0])
@pytest.mark.parametrize("gamma", [1, 2, 5, 10, 12])
def test_closed_form_equals_geometric_series(alpha, gamma):
    # the definition: expected accepted tokens = sum_{k=0}^{gamma} alpha^k
    series = math.fsum(alpha ** k for k in range(gamma + 1))
    t_d, t_t = 0.7, 3.3
    want = series / (gamma * t_d + t_t)
    assert ko.tpt_value(alpha, gamma, t_d, t_t) == pytest.approx(want, rel=1e-9)


def test_limits():
    for gamma in range(1, 13):
        assert ko.tpt_value(0.0, gamma, 2.0, 7.0) == pytest.approx(1.0 / (gamma * 2.0 + 7.0))
        assert ko.tpt_value(1.0, gamma, 2.0, 7.0) == pytest.approx((gamma + 1) / (gamma * 2.0 + 7.0))
        # continuity across the series/closed-form switch at 1 - alpha = 1e-6
        lo = ko.tpt_value(1 - 1.0000001e-6, gamma, 2.0, 7.0)
        hi = ko.tpt_value(1 - 0.9999999e-6, gamma, 2.0, 7.0)
        assert lo == pytest.approx(hi, rel=1e-8)


def test_grid_known_answers():
    # free drafting (t_draft = 0) with alpha > 0: TPT grows with gamma -> gamma_max
    b, g, v = ko.tpt_select(np.array([0.5]), np.array([0.0]), np.array([True]), 4.0, 1, 10)
    assert (b, g) == (0, 10)
    # alpha = 0: every extra draft token only costs -> gamma_min
    b, g, v = ko.tpt_select(np.array([0.0]), np.array([1.0]), np.array([True]), 4.0, 2, 10)
    assert (b, g) == (0, 2) and v == pytest.approx(1.0 / 6.0)
    # identical budgets tie -> the smaller budget wins; invalid budgets are ignored
    alpha = np.array([0.9, 0.7, 0.7, 0.99])
    t_d = np.array([1.0, 1.0, 1.0, 1.0])
    valid = np.array([False, True, True, False])
    b, g, v = ko.tpt_select(alpha, t_d, valid, 4.0, 1, 8)
    assert b == 1
    # no valid budget
    assert ko.tpt_select(alpha, t_d, np.zeros(4, bool), 4.0, 1, 8)[0] == -1


def test_grid_optimum_by_calculus():
    # For fixed alpha the gamma maximising G(gamma)/(gamma t_d + t_t) is where the marginal
    # accepted token alpha^(gamma+1) stops paying for t_d: check the pick is a local max.
    rng = np.random.default_rng(5)
    for _ in range(50):
        a = float(rng.uniform(0.05, 0.98))
        td, tt = float(rng.uniform(0.05, 2)), float(rng.uniform(1, 10))
        b, g, v = ko.tpt_select(np.array([a]), np.array([td]), np.array([True]), tt, 1, 30)
        f = lambda k: ko.tpt_value(a, k, td, tt)
        if 1 < g < 30:
            assert f(g) >= f(g - 1) and f(g) >= f(g + 1)

"""Lemma 4.1 (cosine margin => same greedy token) checked on oracle states.

The review (referee major comment 2, minor comment 3, circularity check) gives the lemma's
ingredients: equal-norm states x, x', the LM head's logit margin xi at x, max_j |w_i* - w_j|,
and a Cauchy-Schwarz argument.  Written out: for every j != i*,
    (w_i* - w_j) . x' >= xi - |w_i* - w_j| |x' - x|,   |x' - x|^2 = 2 |x|^2 (1 - cos),
so cos(x, x') > 1 - xi^2 / (2 |x|^2 D^2), D = max_j |w_i* - w_j|, implies the same argmax.
"""
import numpy as np
import pytest

from tests.helpers import Problem
from workloads import WORKLOADS, synth


def _bound(W, x):
    logits = W @ x
    top = int(np.argmax(logits))
    others = np.delete(np.arange(W.shape[0]), top)
    xi = float(logits[top] - logits[others].max())
    D = float(np.max(np.linalg.norm(W[top][None, :] - W[others], axis=1)))
    return top, 1.0 - xi * xi / (2.0 * float(x @ x) * D * D), D


@pytest.fixture(scope="module")
def tiny():
    return Problem(WORKLOADS["tiny"], seed=0)


def test_lemma_on_dp_states(tiny):
    res = tiny.oracle()
    W = synth.lm_head(tiny.wl, 4096).astype(np.float64)
    x = res.dp.ref.astype(np.float64)
    top, thr, _ = _bound(W, x)
    inside = agree_out = total_out = 0
    for b in np.nonzero(res.dp.valid)[0]:
        xp = res.dp.states[b].astype(np.float64)
        xp *= np.linalg.norm(x) / np.linalg.norm(xp)
        cos = float(xp @ x) / float(x @ x)
        same = int(np.argmax(W @ xp)) == top
        if cos > thr:
            inside += 1
            assert same, (b, cos, thr)
        else:
            total_out += 1
            agree_out += same
    print(f"\n[lemma 4.1] threshold={thr:.6f} inside={inside} outside={total_out} "
          f"agree_outside={agree_out}")


def test_lemma_tight_pairs():
    """Pairs built just inside the bound in the worst direction keep the argmax; the same
    construction well outside the bound flips it (the condition is not vacuous)."""
    rng = np.random.default_rng(0)
    d, V = 64, 512
    W = rng.standard_normal((V, d)) * 0.02
    x = rng.standard_normal(d)
    top, thr, D = _bound(W, x)
    logits = W @ x
    nx = np.linalg.norm(x)
    flips_outside = 0
    for j in np.argsort(logits)[::-1][1:20]:
        u = W[j] - W[top]
        u_perp = u - (u @ x) / (x @ x) * x
        u_perp /= np.linalg.norm(u_perp)
        for c, expect_same in ((thr + 1e-9 * (1 - thr), True), (1 - 25 * (1 - thr), None)):
            c = min(c, 1.0)
            xp = nx * (c * x / nx + np.sqrt(max(0.0, 1 - c * c)) * u_perp)
            same = int(np.argmax(W @ xp)) == top
            if expect_same:
                assert same
            elif not same:
                flips_outside += 1
    assert flips_outside > 0

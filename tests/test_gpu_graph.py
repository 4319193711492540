"""The captured-graph solve path against the eager path, bit for bit.

A solve whose launch configuration matches the previous one replays a captured HIP graph;
inputs travel through the map upload and through device memory the caller rewrites in
place, so every replay must reproduce an eager solve of the same data exactly.
"""
import os

import numpy as np
import pytest

from workloads import WORKLOADS, scaled, synth

pytestmark = pytest.mark.gpu

FIELDS = ("masks", "cos", "valid", "t_draft", "decisions", "margins", "best_budget",
          "best_gamma", "best_tpt", "item_weight")


def _same(a, b):
    for f in FIELDS:
        x, y = getattr(a, f), getattr(b, f)
        if x.dtype.kind == "f":
            assert np.array_equal(x, y, equal_nan=True), f
        else:
            assert np.array_equal(x, y), f


def _solve(prob, graphs, ctxs=None):
    os.environ["KNAPSPEC_GRAPHS"] = "1" if graphs else "0"
    try:
        return prob.solve(flags=3, ctxs=ctxs)
    finally:
        os.environ.pop("KNAPSPEC_GRAPHS", None)


def test_graph_replays_match_eager():
    from workloads.device import DeviceProblem

    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=3, d_model=1024, d_ff=2048, name="graph_t")
    prob = DeviceProblem(wl, 3, ctxs=[700], caps=[1200], max_budgets=64)
    B = 64
    prob.model.solve(prob.seq_args(), B, wl.gamma, flags=3)  # first sight: eager; next: capture
    for rep in range(4):
        # new input values in the same buffers: x0 and the first layer's cache
        prob.set_x0(0, synth.x0(wl, 0, rep + 1, seed=3))
        if rep == 2:
            prob.k_cache[0][0].mul_(-1.0)
        g = prob.model.solve(prob.seq_args(), B, wl.gamma, flags=3)  # graph path (default)
        os.environ["KNAPSPEC_GRAPHS"] = "0"
        try:
            e = prob.model.solve(prob.seq_args(), B, wl.gamma, flags=3)
        finally:
            os.environ.pop("KNAPSPEC_GRAPHS", None)
        _same(g, e)
        print(f"replay {rep}: best=({int(g.best_budget[0])}, {int(g.best_gamma[0])}) ok")
    # a different context length changes the launch configuration (recapture), then back
    g2 = prob.model.solve(prob.seq_args([1100]), B, wl.gamma, flags=3)
    g2 = prob.model.solve(prob.seq_args([1100]), B, wl.gamma, flags=3)
    os.environ["KNAPSPEC_GRAPHS"] = "0"
    try:
        e2 = prob.model.solve(prob.seq_args([1100]), B, wl.gamma, flags=3)
        e3 = prob.model.solve(prob.seq_args(), B, wl.gamma, flags=3)
    finally:
        os.environ.pop("KNAPSPEC_GRAPHS", None)
    _same(g2, e2)
    for _ in range(3):  # eager (new after 1100), capture, replay
        g3 = prob.model.solve(prob.seq_args(), B, wl.gamma, flags=3)
        _same(g3, e3)
    prob.close()

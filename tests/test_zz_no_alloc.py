"""knapspec_solve_static (per-solve device buffers in the library's static scratch, no
allocation) against knapspec_solve on the same inputs: two calls in a row, the second with a
smaller input (fewer budgets, shorter context, another x0), each compared bit for bit with
knapspec_solve's output on the same input (same kernels, deterministic); then a third call with
tau pruning on, whose live-row plan builds its row maps in the static array too.  Also: a model
whose per-solve buffers exceed the static scratch is refused with EINVAL."""
import math

import numpy as np
import pytest

from workloads import WORKLOADS, scaled

pytestmark = pytest.mark.gpu

FIELDS = ("masks", "cos", "valid", "t_draft", "item_weight", "best_budget", "best_gamma",
          "best_tpt", "decisions", "margins")


def same(a, b):
    for f in FIELDS:
        x, y = getattr(a, f), getattr(b, f)
        eq = np.array_equal(x, y, equal_nan=True) if x.dtype.kind == "f" else np.array_equal(x, y)
        assert eq, f


@pytest.mark.parametrize("wl", [
    WORKLOADS["tiny"],
    scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=3, d_model=1024, d_ff=2048, name="bf16_small"),
])
def test_static_scratch_solve_matches_solve(wl):
    from workloads.device import DeviceProblem

    print(f"\n[case] knapspec_solve_static vs knapspec_solve: {wl.name}", flush=True)
    B = 48 if wl.shape.dtype == "bf16" else wl.n_budgets
    prob = DeviceProblem(wl, 0, ctxs=[300], max_budgets=B)
    big = dict(n_budgets=B, flags=3, ctxs=[300])
    small = dict(n_budgets=B // 2 + 3, flags=3, ctxs=[97])
    # first call: the full input; second: a smaller one (the array keeps the first call's
    # contents, which the second must not depend on)
    ref1 = prob.solve(**big)
    st1 = prob.model.solve(prob.seq_args([300]), big["n_budgets"], wl.gamma, -math.inf, -1, 3,
                           static_scratch=True)
    same(st1, ref1)
    x1 = prob.host_x0[0]
    prob.set_x0(0, (x1[::-1] * 1.5).astype(np.float32).copy())
    ref2 = prob.solve(**small)
    st2 = prob.model.solve(prob.seq_args([97]), small["n_budgets"], wl.gamma, -math.inf, -1, 3,
                           static_scratch=True)
    same(st2, ref2)
    assert not np.array_equal(st1.cos[0][: small["n_budgets"]], st2.cos[0])
    ref3 = prob.solve(n_budgets=B, tau=0.5, flags=3, ctxs=[300])
    st3 = prob.model.solve(prob.seq_args([300]), B, wl.gamma, 0.5, -1, 3, static_scratch=True)
    same(st3, ref3)
    assert st3.valid[0].sum() <= ref1.valid[0].sum()  # pruning only removes budgets
    print(f"  static == solve on both calls: picks {(int(st1.best_budget[0]), int(st1.best_gamma[0]))}"
          f" and {(int(st2.best_budget[0]), int(st2.best_gamma[0]))}", flush=True)
    prob.close()


def test_static_scratch_refuses_oversized_model():
    from draft_layer_selection_amd import knapspec as ks
    from workloads.device import DeviceProblem

    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=1, d_model=1024, d_ff=2048, name="wide")
    # 16 sequences x 1024 budgets of d 1024 float32 states alone exceed 64 MiB
    prob = DeviceProblem(wl, 0, ctxs=[10] * 16, max_budgets=1024)
    with pytest.raises(ks.KnapSpecError) as e:
        prob.model.solve(prob.seq_args([10] * 16), 64, wl.gamma, static_scratch=True)
    assert "static scratch" in str(e.value)
    # the regular entry point still works on the same model
    res = prob.solve(n_budgets=64, ctxs=[10] * 16)
    assert res.valid[:, 0].all()
    prob.close()

"""The live-row plan on the GPU: with tau or skip-cap pruning on, every item after the first
gets its rows rebuilt on the device from the previous item's valid flags, so pruned budgets
leave the GEMMs, the attention and its partial results.

* Nothing pruned (tau = -2 lies below every cosine; a skip cap above every prefix weight): the
  live rows are every reachable row, in the host planner's order, and the attention splits are
  the host planner's, so the results are bit-identical to those of the solve that keeps the
  rows planned from reachability (KNAPSPEC_KEEP_PRUNED_ROWS) -- one and several sequences,
  float32 and bfloat16 (head sizes 128 and 64), windows of 1, 2 and 3 tokens, with and
  without the LM-head estimate.
* Everything pruned after the first item (tau = 1.5): only the reference rows stay; results
  are bit-identical too (all budgets invalid).
* Pruned for real (tau = 0.5, a skip cap): both plans pass parity against the oracle's DP
  with the same pruning, one and several sequences, bfloat16 at head size 64 too (4 sequences
  x 200 budgets puts more than 512 rows in every item, so the MLP items get live-row plans
  too); the full Qwen3-1.7B preset and the Llama-3-8B 32K preset at tau = 0.5 against the
  oracle's whole DP.
"""
import math

import numpy as np
import pytest

from tests.test_gpu_parity import run_case
from workloads import WORKLOADS, scaled

pytestmark = pytest.mark.gpu

KEEP = 8  # KNAPSPEC_KEEP_PRUNED_ROWS


def _same(a, b, what):
    if a is None or b is None:
        assert a is None and b is None, what
        return
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype.kind == "f":
        assert np.array_equal(a, b, equal_nan=True), what
    else:
        assert np.array_equal(a, b), what


def _bit_equal(wl, ctxs, tau=-math.inf, cap=-1, window=1, n_budgets=None, seed=0, lm_vocab=0):
    from workloads.device import DeviceProblem

    print(f"\n[case] live rows vs kept rows {wl.name} ctxs={ctxs} tau={tau} cap={cap} "
          f"window={window} B={n_budgets or wl.n_budgets} vocab={lm_vocab}", flush=True)
    prob = DeviceProblem(wl, seed, ctxs=ctxs, window=window,
                         max_budgets=n_budgets or wl.n_budgets, lm_vocab=lm_vocab)
    B = n_budgets or wl.n_budgets
    flags = 3 if window == 1 else 0
    if lm_vocab:
        flags |= prob.ks.KNAPSPEC_ALPHA_LM_HEAD
    live = prob.solve(n_budgets=B, tau=tau, max_skip_weight=cap, flags=flags)
    kept = prob.solve(n_budgets=B, tau=tau, max_skip_weight=cap, flags=flags | KEEP)
    again = prob.solve(n_budgets=B, tau=tau, max_skip_weight=cap, flags=flags)
    for name in ("masks", "cos", "valid", "t_draft", "item_weight", "best_budget",
                 "best_gamma", "best_tpt", "decisions", "margins", "alpha", "tokens_flat"):
        _same(getattr(live, name), getattr(kept, name), name)
        _same(getattr(live, name), getattr(again, name), name + " (repeat)")
    n_valid = int(live.valid.sum())
    print(f"  bit-identical; valid budgets {n_valid}", flush=True)
    prob.close()
    return live


def _bf16_gqa():
    return scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=3, d_model=1024, d_ff=2048,
                  name="bf16_gqa_live")


def _bf16_dh64():
    return scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=3, d_model=512, n_q_heads=8,
                  n_kv_heads=2, head_dim=64, d_ff=1024, name="bf16_dh64_live")


def test_nothing_pruned_tiny_f32():
    res = _bit_equal(WORKLOADS["tiny"], None, tau=-2.0)
    assert res.valid.sum() > 1


def test_nothing_pruned_bf16_three_sequences():
    _bit_equal(_bf16_gqa(), [333, 1000, 77], tau=-2.0, n_budgets=48)


def test_nothing_pruned_bf16_head_dim_64():
    _bit_equal(_bf16_dh64(), [700, 90, 2000], tau=-2.0, n_budgets=64)


def test_nothing_pruned_window3_skip_cap():
    _bit_equal(WORKLOADS["tiny"], [100, 40], cap=10 ** 6, window=3)


def test_nothing_pruned_window_lm_head():
    # the last item's select feeds the LM-head rows at their planned places either way
    _bit_equal(WORKLOADS["tiny"], [130, 60], cap=10 ** 6, window=2, lm_vocab=512)


def test_nothing_pruned_mlp_items_planned_too():
    # 4 sequences x 200 budgets: items hold more than 512 rows, so MLP items get a live-row
    # plan as well (their GEMMs skip m-tiles past the live rows)
    _bit_equal(WORKLOADS["tiny"], [256, 100, 31, 0], tau=-2.0, n_budgets=200)


def test_pruned_parity_mlp_items_planned_too():
    run_case(WORKLOADS["tiny"], ctxs=[256, 100, 31, 0], tau=0.3, n_budgets=200)


def test_nothing_pruned_twenty_sequences():
    # more sequences than the plan kernel has waves: each wave plans several sequences
    ctxs = [(37 * k) % 251 for k in range(20)]
    _bit_equal(WORKLOADS["tiny"], ctxs, tau=-2.0, n_budgets=40)


def test_pruned_parity_twenty_sequences():
    run_case(WORKLOADS["tiny"], ctxs=[(37 * k) % 251 for k in range(20)], tau=0.3, n_budgets=40)


def test_pruned_parity_1024_budgets():
    # the largest budget count: the single-sequence plan holds one budget per thread
    wl = scaled(WORKLOADS["tiny"], n_layers=4, name="tiny_l4_b1024")
    run_case(wl, ctxs=[130], tau=0.3, n_budgets=1024)


def test_everything_pruned_after_first_item():
    res = _bit_equal(_bf16_gqa(), [200, 90], tau=1.5, n_budgets=24)
    assert res.valid.sum() == 0


def test_pruned_parity_tiny_f32_two_sequences():
    wl = scaled(WORKLOADS["tiny"], n_kv_heads=2, name="tiny_gqa_live")
    for flags in (3, 3 | KEEP):
        run_case(wl, ctxs=[130, 47], tau=0.3, cap=6, flags=flags)


def test_pruned_parity_bf16_three_sequences():
    wl = _bf16_gqa()
    for flags in (3, 3 | KEEP):
        run_case(wl, ctxs=[333, 1000, 77], tau=0.5, n_budgets=48, flags=flags)


def test_pruned_parity_bf16_head_dim_64():
    for flags in (3, 3 | KEEP):
        run_case(_bf16_dh64(), ctxs=[700, 90, 2000], tau=0.5, n_budgets=64, flags=flags)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["qwen3_1p7b_4k", "llama3_8b_32k"])
def test_full_preset_tau_half(name):
    from tests.helpers import WidenedLayers
    from tests.test_gpu_fullsize import full_parity
    from workloads.device import DeviceProblem

    wl = WORKLOADS[name]
    print(f"\n[case] {wl.name} full size, tau = 0.5, whole-DP parity", flush=True)
    prob = DeviceProblem(wl, 0, keep_host=True)
    res = prob.solve(tau=0.5, flags=3)
    reach = prob.solve(flags=3)
    # pruning only removes budgets
    assert not np.any(res.valid[0].astype(bool) & ~reach.valid[0].astype(bool))
    print(f"  valid budgets {int(res.valid[0].sum())} of {int(reach.valid[0].sum())} reachable",
          flush=True)
    full_parity(WidenedLayers(prob.host_layers), prob, res, 0, wl, prob.ctxs[0],
                prob.host_x0[0], tau=0.5)
    prob.close()

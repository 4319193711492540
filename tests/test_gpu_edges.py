"""Edge cases of the GPU solve against the oracle (rules P1-P4, tests/parity.py): the smallest
and the largest budget count, a one-layer decoder, multi-query attention (one KV head), a
float32 hidden size that is not a multiple of 64, a skip cap of zero (only the full model
survives), and a one-point gamma grid."""
import numpy as np
import pytest

from tests.test_gpu_parity import run_case
from workloads import WORKLOADS, scaled

pytestmark = pytest.mark.gpu


def test_two_budgets():
    res, reps = run_case(WORKLOADS["tiny"], ctxs=[50], n_budgets=2)
    orc, rep = reps[0]
    assert rep.excused == 0 and np.array_equal(res.masks[0], orc.masks)


def test_largest_budget_count():
    # 1024 budgets: the latency quantum is 1/1023 of the model's latency, so the items weigh
    # 46..82 and most budgets are unreachable; rows per item reach the hundreds
    res, reps = run_case(scaled(WORKLOADS["tiny"], n_layers=4), ctxs=[130], n_budgets=1024)
    orc, rep = reps[0]
    assert rep.excused == 0 and np.array_equal(res.masks[0], orc.masks)
    assert 4 < int(res.valid[0].sum()) < 1024


def test_one_layer_decoder():
    res, reps = run_case(scaled(WORKLOADS["tiny"], n_layers=1), ctxs=[64], n_budgets=8)
    orc, rep = reps[0]
    assert np.array_equal(res.masks[0], orc.masks)


def test_multi_query_attention_bf16():
    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=3, d_model=1024, n_q_heads=8,
                n_kv_heads=1, d_ff=2048, name="bf16_mqa")
    run_case(wl, ctxs=[333], n_budgets=40)


def test_f32_hidden_size_not_multiple_of_64():
    wl = scaled(WORKLOADS["tiny"], n_layers=3, d_model=260, d_ff=224, name="tiny_d260")
    res, reps = run_case(wl, ctxs=[90], n_budgets=24)
    orc, rep = reps[0]
    assert rep.excused == 0 and np.array_equal(res.masks[0], orc.masks)


def test_skip_cap_zero_keeps_only_the_full_model():
    wl = WORKLOADS["tiny"]
    res, reps = run_case(wl, cap=0)
    orc, rep = reps[0]
    # with no skipped weight allowed, the only live cell after the last item is the full set
    assert int(res.valid[0].sum()) == int(orc.dp.valid.sum()) == 1
    b = int(np.nonzero(res.valid[0])[0][0])
    assert b == int(np.sum(orc.w)) and abs(float(res.cos[0][b]) - 1.0) < 1e-6


def test_one_point_gamma_grid():
    wl = scaled(WORKLOADS["tiny"], gamma=(3, 3), name="tiny_gamma3")
    res, reps = run_case(wl)
    assert int(res.best_gamma[0]) == 3 and reps[0][1].same_pick

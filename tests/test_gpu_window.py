"""GPU knapspec_solve with r-token windows and the LM-head acceptance estimate vs the oracle.

* Windows r = 2..8 on the float32 tiny decoder, r = 4 on a bf16 MFMA-path decoder and r = 5
  with the LM-head estimate on the full Qwen3-1.7B preset:
  rules P1-P4 (tests/parity.py) with the oracle's window DP (causal block attention over the
  cache, flattened r x d cosine).
* A model loaded for windows up to 4 solving r = 1 matches the single-token oracle.
* KNAPSPEC_ALPHA_LM_HEAD: every budget's greedy tokens against the oracle's forward of the
  GPU's own mask (rule P5 in tests/parity.py), excusing tokens whose top-2 logit margin is
  inside the band; the TPT pick is the grid's argmax over the returned alphas.
"""
import math

import numpy as np
import pytest

from oracle import knapspec_oracle as ko
from tests.helpers import decoder_shape
from tests.parity import compare, compare_alpha
from workloads import WORKLOADS, scaled

pytestmark = pytest.mark.gpu

BETA = {"f32": 1e-5, "bf16": 2e-3}
# greedy-token band in logit units.  A logit gap l_i - l_j moves by sum_k dx_k (w_ik - w_jk)
# when the normed final state moves by dx.  With a relative state error e per element (bf16
# rows: e ~ 2^-8 after a few rounded items) and LM-head rows N(0, 0.02^2), the typical shift
# is e * sqrt(sum_k x_k^2 (w_ik - w_jk)^2) ~ e * sqrt(d) * 0.028, i.e. ~0.0035 at d = 1024;
# the band is ~14 times that (a statistical band, not a worst-case bound).  float32: 1e-3.
LM_BAND = {"f32": 1e-3, "bf16": 0.05}


def run_window(wl, r, ctx, n_budgets=None, lm_vocab=0, max_window=None, seed=0,
               tau=-math.inf):
    from workloads.device import DeviceProblem

    B = n_budgets or wl.n_budgets
    print(f"\n[case] window r={r} {wl.name} L={wl.shape.n_layers} d={wl.shape.d_model} "
          f"dtype={wl.shape.dtype} ctx={ctx} B={B} vocab={lm_vocab}", flush=True)
    prob = DeviceProblem(wl, seed, ctxs=[ctx], keep_host=True, max_budgets=B,
                         window=max_window or r, lm_vocab=lm_vocab)
    if max_window and r != prob.window:  # a smaller window than the model's capacity
        from workloads import synth
        prob.window = r
        x = synth.x0(wl, 0, 0, seed) if r == 1 else synth.x0_window(wl, r, 0, 0, seed)
        prob.host_x0[0] = x
        prob.x0[0] = prob.torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    flags = 3 | (prob.ks.KNAPSPEC_ALPHA_LM_HEAD if lm_vocab else 0)
    res = prob.solve(n_budgets=B, flags=flags, tau=tau)
    beta = BETA[wl.shape.dtype]
    n_items = 2 * wl.shape.n_layers
    lat = {"attn_base": wl.latency.attn_base, "attn_per_token": wl.latency.attn_per_token,
           "mlp": wl.latency.mlp, "fixed": wl.latency.fixed}
    items = ko.DecoderItems(decoder_shape(wl), prob.host_layers, prob.host_kv[0], ctx,
                            cache_widened=True)
    x0 = prob.host_x0[0]
    orc = ko.solve(decoder_shape(wl), None, None, x0, ctx, lat, B, wl.gamma, tau=tau,
                   apply_item=items, w_lm=prob.host_lm if lm_vocab else None)
    rep = compare(orc, res, 0, beta, items, x0, wl.gamma, n_items)
    print(f"  {rep.line()}", flush=True)
    assert rep.mismatched_clean == 0
    assert rep.p2_max_err <= beta
    assert rep.p3_bad == 0
    if not lm_vocab:
        assert rep.p4_ok
    else:
        arep = compare_alpha(res, 0, items, x0, prob.host_lm, wl.shape.rms_eps,
                             LM_BAND[wl.shape.dtype], n_items)
        print(f"  alpha: {arep.line()}", flush=True)
        assert arep.mismatched_tokens == 0
        assert arep.alpha_mismatch == 0
        # the pick is the TPT grid's argmax over the returned alphas (ties: smaller b, gamma)
        bb, bg, bt = ko.tpt_select(res.alpha[0].astype(np.float64), res.t_draft[0],
                                   res.valid[0].astype(bool), orc.t_target, *wl.gamma)
        assert (bb, bg) == (int(res.best_budget[0]), int(res.best_gamma[0]))
    prob.close()
    return res, orc, rep


@pytest.mark.parametrize("r", [2, 3, 8])
def test_tiny_f32_windows(r):
    res, orc, rep = run_window(WORKLOADS["tiny"], r, ctx=130)
    assert rep.excused == 0
    assert np.array_equal(res.masks[0], orc.masks)


def test_tiny_f32_window_without_cache():
    run_window(WORKLOADS["tiny"], 4, ctx=0)


def test_single_token_on_window_capable_model():
    res, orc, rep = run_window(WORKLOADS["tiny"], 1, ctx=77, max_window=4)
    assert rep.excused == 0
    assert np.array_equal(res.masks[0], orc.masks)


def test_bf16_window_mfma_path():
    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=4, d_model=1024, d_ff=2048,
                name="qwen_like_window")
    run_window(wl, 4, ctx=1000, n_budgets=64)


def test_bf16_window_head_dim_64():
    # head size 64 on the MFMA kernel with r = 4 window rows per state
    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=3, d_model=512, n_q_heads=8,
                n_kv_heads=2, head_dim=64, d_ff=1024, name="dh64_window")
    run_window(wl, 4, ctx=900, n_budgets=48)


def test_tiny_f32_window_lm_head_alpha():
    res, orc, rep = run_window(WORKLOADS["tiny"], 3, ctx=130, lm_vocab=512)
    # float32, no near-ties: the same masks, so the same alphas and the same pick
    assert np.array_equal(res.masks[0], orc.masks)
    assert np.allclose(res.alpha[0].astype(np.float64), orc.alpha, rtol=0, atol=1e-6)
    assert (int(res.best_budget[0]), int(res.best_gamma[0])) == (orc.best_budget, orc.best_gamma)


def test_tiny_f32_window_lm_head_alpha_pruned():
    # tau pruning on: the live-row plan drops pruned budgets from every item after the first,
    # while the last item's rows still feed the LM-head pass at their planned places
    res, orc, rep = run_window(WORKLOADS["tiny"], 3, ctx=130, lm_vocab=512, tau=0.3)
    assert np.array_equal(res.masks[0], orc.masks)
    assert np.array_equal(res.valid[0].astype(bool), orc.dp.valid)
    assert np.allclose(res.alpha[0].astype(np.float64), orc.alpha, rtol=0, atol=1e-6)


def test_bf16_window_lm_head_alpha():
    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=3, d_model=1024, d_ff=2048,
                name="qwen_like_lm")
    run_window(wl, 4, ctx=700, n_budgets=48, lm_vocab=4096)


def test_qwen3_1p7b_full_preset_window_lm_head():
    # the full Qwen3-1.7B preset (28 layers, n = 4096, 128 budgets) with r = 5 token states
    # (one from each of the last m = 5 steps) and the LM-head estimate over 32768 rows
    run_window(WORKLOADS["qwen3_1p7b_4k"], 5, ctx=4096, lm_vocab=32768)

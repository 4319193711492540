"""GPU knapspec_solve with the beam variant of the DP (top-k states per cell) vs the oracle.

* beam 1 on a model sized for beams is the one-state DP (masks bit-equal on float32);
* beams 2, 4 and 8 on the float32 tiny decoder: each budget's best set equals the oracle
  beam's (rules P2-P4 of tests/parity.py, masks bit-equal);
* a beam of 8 on a 3-layer decoder whose same-weight subset counts are at most 8 keeps every
  subset: each budget's best set is the best subset of that weight by enumeration;
* a bf16 MFMA-path decoder at beam 4: P2 (the reported cosine is that of the returned set)
  and the valid budgets; the best-set agreement with the oracle is reported.
"""
import math

import numpy as np
import pytest

from oracle import knapspec_oracle as ko
from tests.helpers import decoder_shape
from tests.parity import compare
from workloads import WORKLOADS, scaled

pytestmark = pytest.mark.gpu

BETA = {"f32": 1e-5, "bf16": 2e-3}


def run_beam(wl, beam, ctx, n_budgets=None, per_item=None, max_beam=None, window=1):
    from workloads.device import DeviceProblem

    B = n_budgets or wl.n_budgets
    print(f"\n[case] beam={beam} {wl.name} L={wl.shape.n_layers} d={wl.shape.d_model} "
          f"dtype={wl.shape.dtype} ctx={ctx} B={B} per_item={per_item} r={window}", flush=True)
    prob = DeviceProblem(wl, 0, ctxs=[ctx], keep_host=True, max_budgets=B,
                         max_beam=max_beam or beam, window=window)
    lat = wl.latency
    if per_item is not None:
        prob.model.set_latency(lat.attn_base, lat.attn_per_token, lat.mlp, lat.fixed,
                               per_item=per_item)
    res = prob.solve(n_budgets=B, beam=beam, flags=3 if beam == 1 else 0)
    n_items = 2 * wl.shape.n_layers
    latd = {"attn_base": lat.attn_base, "attn_per_token": lat.attn_per_token, "mlp": lat.mlp,
            "fixed": lat.fixed}
    items = ko.DecoderItems(decoder_shape(wl), prob.host_layers, prob.host_kv[0], ctx,
                            cache_widened=True)
    x0 = prob.host_x0[0]
    orc = ko.solve(decoder_shape(wl), None, None, x0, ctx, latd, B, wl.gamma, per_item=per_item,
                   apply_item=items, beam=beam)
    beta = BETA[wl.shape.dtype]
    rep = compare(orc, res, 0, beta, items, x0, wl.gamma, n_items)
    same = np.all(ko.unpack_masks(res.masks[0], n_items) == orc.dp.bits, axis=1) & orc.dp.valid
    print(f"  {rep.line()} best-set agreement {int(same.sum())}/{int(orc.dp.valid.sum())}",
          flush=True)
    assert rep.p2_max_err <= beta
    assert np.array_equal(res.valid[0].astype(bool), orc.dp.valid)
    prob.close()
    return res, orc, rep, items, x0


def test_beam_one_on_beam_capable_model():
    res, orc, rep, _, _ = run_beam(WORKLOADS["tiny"], 1, ctx=130, max_beam=4)
    assert rep.mismatched_clean == 0 and rep.p4_ok
    assert np.array_equal(res.masks[0], orc.masks)


@pytest.mark.parametrize("beam", [2, 4, 8])
def test_tiny_f32_beams(beam):
    res, orc, rep, _, _ = run_beam(WORKLOADS["tiny"], beam, ctx=130)
    assert np.array_equal(res.masks[0], orc.masks)
    assert rep.p4_ok and rep.same_pick


def test_tiny_f32_beam_with_window():
    res, orc, rep, _, _ = run_beam(WORKLOADS["tiny"], 3, ctx=60, window=2)
    assert np.array_equal(res.masks[0], orc.masks)


def test_beam_eight_is_exhaustive_on_small_decoder():
    wl = scaled(WORKLOADS["tiny"], n_layers=3, name="beam_exhaustive")
    per_item = [4.0, 4.0, 8.0, 2.0, 4.0, 1.0]   # weights 3,3,6,1,3,1 at B = 17: <= 8 subsets
    res, orc, rep, items, x0 = run_beam(wl, 8, ctx=50, n_budgets=17, per_item=per_item)
    n_items = 6
    ids, cos_all = ko.brute_force(items, n_items, x0)
    w = res.item_weight[0]
    weight = np.array([sum(int(w[i]) for i in range(n_items) if (s >> i) & 1) for s in ids])
    gbits = ko.unpack_masks(res.masks[0], n_items)
    for b in range(17):
        sel = weight == b
        assert bool(res.valid[0][b]) == bool(sel.any())
        if not sel.any():
            continue
        best = int(ids[sel][np.argmax(cos_all[sel])])
        gid = int(sum(1 << i for i in range(n_items) if gbits[b, i]))
        assert gid == best, (b, gid, best)
        assert float(res.cos[0][b]) == pytest.approx(float(cos_all[sel].max()), abs=1e-5)


def test_bf16_beam_mfma_path():
    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=3, d_model=1024, d_ff=2048,
                name="qwen_like_beam")
    run_beam(wl, 4, ctx=700, n_budgets=48)


def test_bf16_beam_head_dim_64():
    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=3, d_model=512, n_q_heads=8,
                n_kv_heads=2, head_dim=64, d_ff=1024, name="dh64_beam")
    run_beam(wl, 4, ctx=700, n_budgets=48)


def test_qwen3_1p7b_full_preset_beam4():
    # the full Qwen3-1.7B preset (28 layers, n = 4096, 128 budgets) keeping 4 states per cell
    run_beam(WORKLOADS["qwen3_1p7b_4k"], 4, ctx=4096)

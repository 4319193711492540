"""GPU knapspec_solve vs the CPU oracle on seeded inputs (rules P1-P4, tests/parity.py).

Sizes here let the oracle finish in seconds while spanning several GEMM/attention tiles and
ragged tails; the full-size presets are in test_gpu_fullsize.py.
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


def run_case(wl, seed=0, ctxs=None, tau=-math.inf, cap=-1, n_budgets=None, per_item=None,
             flags=3, prepare=None):
    """Solve on the GPU and compare with the oracle's DP (P1-P4).  ``prepare(prob)`` may edit
    the inputs (host and device copies alike) before the solve."""
    from workloads.device import DeviceProblem

    print(f"\n[case] {wl.name} L={wl.shape.n_layers} d={wl.shape.d_model} "
          f"hq/hkv={wl.shape.n_q_heads}/{wl.shape.n_kv_heads} dh={wl.shape.head_dim} "
          f"dtype={wl.shape.dtype} ctxs={ctxs} B={n_budgets or wl.n_budgets} tau={tau} cap={cap} "
          f"flags={flags}", flush=True)
    prob = DeviceProblem(wl, seed, ctxs=ctxs, keep_host=True,
                         max_budgets=n_budgets or wl.n_budgets)
    if prepare is not None:
        prepare(prob)
    B = n_budgets or wl.n_budgets
    res = prob.solve(n_budgets=B, tau=tau, max_skip_weight=cap, flags=flags)
    beta = BETA[wl.shape.dtype]
    n_items = 2 * wl.shape.n_layers
    lat = {"attn_base": wl.latency.attn_base, "attn_per_token": wl.latency.attn_per_token,
           "mlp": wl.latency.mlp, "fixed": wl.latency.fixed}
    reports = []
    for q in range(len(prob.ctxs)):
        items = ko.DecoderItems(decoder_shape(wl), prob.host_layers, prob.host_kv[q],
                                prob.ctxs[q], cache_widened=True)
        orc = ko.solve(decoder_shape(wl), None, None, prob.host_x0[q], prob.ctxs[q], lat, B,
                       wl.gamma, tau=tau, skip_cap=cap, apply_item=items)
        rep = compare(orc, res, q, beta, items, prob.host_x0[q], wl.gamma, n_items)
        print(f"  seq {q} ctx={prob.ctxs[q]}: {rep.line()}", flush=True)
        assert rep.mismatched_clean == 0
        assert rep.p2_max_err <= beta
        assert rep.p3_bad == 0
        assert rep.p4_ok
        reports.append((orc, rep))
    prob.close()
    return res, reports


def test_tiny_f32_full_preset():
    res, reps = run_case(WORKLOADS["tiny"])
    orc, rep = reps[0]
    # float32 everywhere: no near-ties in this preset, so everything must match exactly
    assert rep.excused == 0
    assert np.array_equal(res.masks[0], orc.masks)
    assert rep.same_pick


def test_tiny_f32_fixed_latency_interior_pick():
    # A per-pass latency `fixed` equal to one MLP item's makes the empty draft cost something,
    # so the TPT pick moves off the (b = 0, gamma = gamma_max) corner into the grid (the
    # oracle picks b = 5, gamma = 1 on seed 0); the float32 path must reproduce it exactly.
    from workloads.configs import LatencyModel

    wl = scaled(WORKLOADS["tiny"], latency=LatencyModel(1.0, 0.01, 2.0, 2.0),
                name="tiny_fixed2")
    res, reps = run_case(wl)
    orc, rep = reps[0]
    assert rep.excused == 0 and rep.same_pick
    assert np.array_equal(res.masks[0], orc.masks)
    assert 0 < orc.best_budget < wl.n_budgets - 1
    assert (int(res.best_budget[0]), int(res.best_gamma[0])) == (orc.best_budget, orc.best_gamma)
    assert np.allclose(res.t_draft[0][orc.dp.valid], orc.t_draft[orc.dp.valid], rtol=0, atol=1e-12)
    assert float(res.best_tpt[0]) == pytest.approx(orc.best_tpt, rel=1e-6)


@pytest.mark.parametrize("ctx", [0, 1, 77, 300])
def test_tiny_f32_context_edges(ctx):
    run_case(WORKLOADS["tiny"], ctxs=[ctx])


def test_tiny_f32_gqa_and_pruning():
    wl = scaled(WORKLOADS["tiny"], n_kv_heads=2, n_layers=5)
    run_case(wl, ctxs=[130])
    run_case(wl, ctxs=[130], tau=0.5)
    run_case(wl, ctxs=[130], cap=6)


def test_tiny_f32_tau_above_one():
    res, _ = run_case(WORKLOADS["tiny"], tau=1.5)
    assert not res.valid.any()
    assert int(res.best_budget[0]) == -1


def test_bf16_small_mfma_path():
    # Qwen3-1.7B head layout (16 q / 8 kv heads of 128) on a narrow 4-layer decoder;
    # ctx 1000 is not a multiple of the 64-key tile and splits over several workgroups.
    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=4, d_model=1024, d_ff=2048,
                name="qwen_like_small")
    run_case(wl, ctxs=[1000], n_budgets=64)


def _keys_scaled_by_tile_pairs(low: float, high: float):
    """Scale the cached keys of 64-key tile t by ``low`` for even t and ``high`` for odd t
    (powers of two: exact in bf16), in the oracle's copy and on the device alike."""
    def prepare(prob):
        import torch

        from workloads import synth
        for q in range(len(prob.ctxs)):
            for l, (kb, vb) in enumerate(prob.host_kv[q]):
                pos = np.arange(kb.shape[1])
                f = np.where((pos // 64) % 2 == 1, high, low).astype(np.float32)
                nb = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(kb) * f[None, :, None])
                prob.host_kv[q][l] = (nb, vb)
                dev = torch.from_numpy(np.ascontiguousarray(nb)).view(torch.bfloat16)
                prob.k_cache[q][l].copy_(dev.to("cuda"))
        torch.cuda.synchronize()
    return prepare


def test_bf16_reference_raised_inside_splits():
    # keys of even 64-key tiles scaled by 1/2, of odd tiles by 8: a context split that starts
    # on an even tile sets its reference there, and its next tile scores ~16 above it in the
    # exponent's units (the presets' N(0,1) caches stay within the allowed 8), so the attention
    # raises the reference inside the split -- O, l and the tile's scores shifted, the C
    # operand of the next tile's first score MFMA reset -- at head sizes 128 and 64
    for dh, hq, hkv in ((128, 16, 8), (64, 16, 4)):
        wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=2, d_model=1024, n_q_heads=hq,
                    n_kv_heads=hkv, head_dim=dh, d_ff=2048, name=f"bf16_raise_dh{dh}")
        run_case(wl, ctxs=[6000], n_budgets=48, prepare=_keys_scaled_by_tile_pairs(0.5, 8.0))


def test_bf16_several_query_blocks():
    # GQA group of 4 with up to 116 rows per attention item: a KV head's 4*M query rows span
    # two 256-row blocks from M = 65 on, spread evenly over them (e.g. 260 rows as 160 + 100)
    wl = scaled(WORKLOADS["llama3_8b_32k"], n_layers=12, d_model=1024, n_q_heads=8,
                n_kv_heads=2, d_ff=2048, name="llama_like_qblocks")
    run_case(wl, ctxs=[300], n_budgets=128)


def test_bf16_head_dim_64():
    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=3, d_model=512, n_q_heads=8,
                n_kv_heads=2, head_dim=64, d_ff=1024, name="bf16_dh64")
    run_case(wl, ctxs=[200], n_budgets=40)


def test_bf16_head_dim_64_query_blocks_and_splits():
    # head size 64 on the MFMA kernel: a GQA group of 4 with up to 96 rows per item puts a KV
    # head's query rows in two 256-row blocks; a context of 3000 (47 key tiles, the last one
    # ragged) splits over several workgroups; 450 and an empty cache share the solve
    wl = scaled(WORKLOADS["llama3_8b_32k"], n_layers=4, d_model=1024, n_q_heads=16,
                n_kv_heads=4, head_dim=64, d_ff=2048, name="bf16_dh64_qblocks")
    run_case(wl, ctxs=[3000, 450, 0], n_budgets=96)


def test_bf16_multi_sequence():
    wl = scaled(WORKLOADS["llama3_8b_x16"], n_layers=3, d_model=512, n_q_heads=8,
                n_kv_heads=2, d_ff=1024, n_seqs=3, ctx_range=None, name="multi_small")
    run_case(wl, ctxs=[0, 700, 2100], n_budgets=48)


def test_determinism():
    from workloads.device import DeviceProblem

    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=3, d_model=1024, d_ff=2048)
    prob = DeviceProblem(wl, 1, ctxs=[513], max_budgets=96)
    a = prob.solve(n_budgets=96, flags=3)
    b = prob.solve(n_budgets=96, flags=3)
    for f in ("masks", "cos", "valid", "decisions", "margins", "best_budget", "best_gamma"):
        x, y = getattr(a, f), getattr(b, f)
        assert np.array_equal(x, y, equal_nan=True) if x.dtype.kind == "f" else np.array_equal(x, y), f
    prob.close()


def test_qwen3_1p7b_full_preset():
    run_case(WORKLOADS["qwen3_1p7b_4k"])

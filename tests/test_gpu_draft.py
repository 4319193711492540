"""GPU knapspec_draft_verify (masked draft step + verification pass) vs the oracle.

Tokens are compared in order up to the first position where the oracle's top-2 logit gap is
inside the band (from there on the inputs of later tokens may legitimately differ): draft
tokens y_t, and verification tokens z_t for every t whose inputs (x0, e(y_0) .. e(y_{t-1}))
agree.  With every item executed the draft is the target model and all gamma draft tokens
must be accepted.
"""
import numpy as np
import pytest

from oracle import knapspec_oracle as ko
from tests.helpers import decoder_shape
from workloads import WORKLOADS, scaled

pytestmark = pytest.mark.gpu

BAND = {"f32": 1e-3, "bf16": 0.05}  # logit units, as for the LM-head acceptance estimate


def _compare(gpu, orc, band):
    k = 0  # draft tokens agree on [0, k)
    while k < len(orc.draft) and orc.draft_margin[k] >= band:
        assert int(gpu["draft"][k]) == int(orc.draft[k]), ("draft", k)
        k += 1
    for t in range(k + 1):
        if orc.verify_margin[t] >= band:
            assert int(gpu["verify"][t]) == int(orc.verify[t]), ("verify", t)
    return k


def run_draft(wl, ctx, gamma, vocab, masks, seed=0):
    from workloads.device import DeviceProblem

    print(f"\n[case] draft/verify {wl.name} L={wl.shape.n_layers} d={wl.shape.d_model} "
          f"dtype={wl.shape.dtype} ctx={ctx} gamma={gamma} vocab={vocab}", flush=True)
    prob = DeviceProblem(wl, seed, ctxs=[ctx], caps=[ctx + gamma + 1], keep_host=True,
                         lm_vocab=vocab)
    n_items = 2 * wl.shape.n_layers
    res = prob.solve(n_budgets=wl.n_budgets)
    out = []
    for name, bits in masks(n_items, res):
        mask = ko.pack_masks(bits[None])[0]
        gpu = prob.model.draft_verify(prob.seq_args()[0], mask, gamma)
        orc = ko.draft_verify(decoder_shape(wl), prob.host_layers, prob.host_kv[0],
                              prob.host_x0[0], ctx, bits, gamma, prob.host_lm)
        k = _compare(gpu, orc, BAND[wl.shape.dtype])
        print(f"  {name}: draft {gpu['draft'].tolist()} verify {gpu['verify'].tolist()} "
              f"accepted {gpu['accepted']} (oracle {orc.accepted}); compared {k}/{gamma}; "
              f"draft {gpu['draft_us']:.0f} us verify {gpu['verify_us']:.0f} us", flush=True)
        out.append((name, gpu, orc, k))
    prob.close()
    return out


def _masks(n_items, res):
    full = np.ones(n_items, bool)
    b = int(res.best_budget[0])
    pick = ko.unpack_masks(res.masks[0][b:b + 1], n_items)[0] if b >= 0 else full
    half = np.zeros(n_items, bool)
    half[: n_items // 2] = True
    return [("full", full), ("pick", pick), ("half", half), ("empty", np.zeros(n_items, bool))]


def test_tiny_f32_draft_verify():
    out = run_draft(WORKLOADS["tiny"], 130, 4, 512, _masks)
    for name, gpu, orc, k in out:
        assert k == 4, name  # float32: no near-ties, every token compared
        assert gpu["accepted"] == orc.accepted
        if name == "full":
            assert gpu["accepted"] == 4


def test_tiny_f32_longest_block():
    wl = scaled(WORKLOADS["tiny"], n_layers=4, name="draft_long")
    out = run_draft(wl, 40, 15, 256, lambda n, r: [("full", np.ones(n, bool))])
    assert out[0][1]["accepted"] == 15


def test_bf16_draft_verify():
    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=3, d_model=1024, d_ff=2048,
                name="qwen_like_draft")
    out = run_draft(wl, 700, 7, 4096, _masks)
    assert any(k > 0 for _, _, _, k in out)


def test_bf16_draft_verify_head_dim_64():
    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=3, d_model=512, n_q_heads=8,
                n_kv_heads=2, head_dim=64, d_ff=1024, name="dh64_draft")
    out = run_draft(wl, 500, 5, 2048, _masks)
    assert any(k > 0 for _, _, _, k in out)


def test_repeated_calls_replay_the_captured_graph():
    # eager, capture, then replays of the same configuration: identical tokens every time
    from workloads.device import DeviceProblem

    wl = WORKLOADS["tiny"]
    prob = DeviceProblem(wl, 0, ctxs=[77], caps=[77 + 6], keep_host=True, lm_vocab=512)
    n_items = 2 * wl.shape.n_layers
    bits = np.zeros(n_items, bool)
    bits[::3] = True
    mask = ko.pack_masks(bits[None])[0]
    runs = [prob.model.draft_verify(prob.seq_args()[0], mask, 5) for _ in range(4)]
    orc = ko.draft_verify(decoder_shape(wl), prob.host_layers, prob.host_kv[0], prob.host_x0[0],
                          77, bits, 5, prob.host_lm)
    for r in runs:
        assert np.array_equal(r["draft"], orc.draft)
        assert np.array_equal(r["verify"], orc.verify)
        assert r["accepted"] == orc.accepted
    print(f"\n  draft us per call: {[round(r['draft_us']) for r in runs]}", flush=True)
    prob.close()


def test_qwen3_1p7b_full_preset_draft_verify():
    # the full Qwen3-1.7B preset (28 layers, n = 4096) with its DP pick, gamma = 8 (the largest
    # draft length of the preset's grid) and an LM head of 32768 rows
    out = run_draft(WORKLOADS["qwen3_1p7b_4k"], 4096, 8, 32768, _masks)
    assert any(k > 0 for _, _, _, k in out)
    full = [o for o in out if o[0] == "full"][0]
    # every item executed: the draft is the target; tokens compared up to the first near-tie
    assert full[1]["accepted"] >= full[3]

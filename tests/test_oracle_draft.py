"""Pins for the oracle's masked draft step and verification pass (draft_verify).

* Every item executed: the draft is the target model, so each draft token equals the
  verification's token at its position (accepted = gamma) -- the verification block is
  checked against token-by-token decoding by the window pins, and the draft against it here.
* No item executed: every draft state is the previous token's embedding, so the draft is the
  greedy chain through the LM head alone (checked by hand).
* The caches passed in are not modified.
"""
import numpy as np

from oracle import knapspec_oracle as ko
from tests.helpers import decoder_shape
from workloads import WORKLOADS, scaled, synth


def _setup(n_layers=3, ctx=30, gamma=4):
    wl = scaled(WORKLOADS["tiny"], n_layers=n_layers, name="draft_t")
    layers = [synth.layer_weights(wl, l, 0) for l in range(n_layers)]
    kv = [synth.kv_cache(wl, l, 0, ctx + gamma + 1, 0) for l in range(n_layers)]
    x0 = synth.x0(wl, 0, 0, 0)
    W = synth.lm_head(wl, vocab=256)
    return wl, layers, kv, x0, W


def test_full_mask_draft_is_accepted():
    wl, layers, kv, x0, W = _setup()
    n = 2 * wl.shape.n_layers
    before = [(k.copy(), v.copy()) for k, v in kv]
    dv = ko.draft_verify(decoder_shape(wl), layers, kv, x0, 30, np.ones(n, bool), 4, W)
    assert dv.accepted == 4
    assert np.array_equal(dv.draft, dv.verify[:4])
    assert np.all(dv.draft_margin > 1e-4)  # not a near-tie: the equality is not by luck
    for (k, v), (k0, v0) in zip(kv, before):
        assert np.array_equal(k, k0) and np.array_equal(v, v0)


def test_empty_mask_draft_is_the_lm_head_chain():
    wl, layers, kv, x0, W = _setup()
    n = 2 * wl.shape.n_layers
    dv = ko.draft_verify(decoder_shape(wl), layers, kv, x0, 30, np.zeros(n, bool), 4, W)
    x = x0.astype(np.float64)
    for t in range(4):
        xn = x / np.sqrt(np.mean(x * x) + wl.shape.rms_eps)
        tok = int(np.argmax(W.astype(np.float64) @ xn))
        assert dv.draft[t] == tok
        x = W[tok].astype(np.float64)
    assert 0 <= dv.accepted <= 4

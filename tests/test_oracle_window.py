"""Pins for the oracle's r-token window (states of r tokens) and the LM-head acceptance
estimate.

* A window of r tokens run through an Attention item as one causal block equals decoding
  the tokens one at a time, each token's key/value appended to the cache before the next
  (the defining property of causal attention, checked against the single-token item, which
  has its own scalar-loop pins).
* A window token never depends on later window tokens.
* The window DP keeps budget 0 at x0, its candidate sets reproduce their cosines when
  re-run, and no candidate beats the best subset of its weight found by enumeration.
* greedy_tokens is the argmax of RMSNorm'd logits (loop check); alpha_lm_head is 1 for the
  full-model state, counts matches of planted greedy tokens, and lies on {0, 1/r, ..., 1}.
"""
import math

import numpy as np
import pytest

from oracle import knapspec_oracle as ko
from tests.helpers import decoder_shape
from workloads import WORKLOADS, scaled, synth


def _shape(**kw):
    base = dict(n_layers=1, d_model=32, n_q_heads=4, n_kv_heads=2, head_dim=8, d_ff=48,
                rms_eps=1e-5, rope_theta=1e4)
    base.update(kw)
    return ko.DecoderShape(**base)


def _weights(s, rng, sigma=0.2):
    q_dim = s.n_q_heads * s.head_dim
    return {
        "w_qkv": (rng.standard_normal(((s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim,
                                       s.d_model)) * sigma).astype(np.float32),
        "w_o": (rng.standard_normal((s.d_model, q_dim)) * sigma).astype(np.float32),
    }


def _kv_of_tokens(X, w, ctx, s):
    """Rotated key and value of each window token (token t at position ctx + t)."""
    M, r, d = X.shape
    hq, hkv, dh = s.n_q_heads, s.n_kv_heads, s.head_dim
    xn = ko.rmsnorm(X, s.rms_eps)
    kv = xn @ w["w_qkv"].T
    k = kv[:, :, hq * dh:(hq + hkv) * dh].reshape(M, r, hkv, dh).copy()
    v = kv[:, :, (hq + hkv) * dh:].reshape(M, r, hkv, dh)
    for t in range(r):
        c, sn = ko.rope_cos_sin(ctx + t, dh, s.rope_theta)
        k[:, t] = ko.rope(k[:, t], c, sn)
    return k, v


@pytest.mark.parametrize("hq,hkv,ctx,r", [(4, 2, 5, 3), (4, 4, 0, 4), (4, 1, 9, 2), (2, 2, 3, 1)])
def test_window_equals_incremental_decoding(hq, hkv, ctx, r):
    s = _shape(n_q_heads=hq, n_kv_heads=hkv)
    rng = np.random.default_rng(100 + 10 * hq + hkv + ctx + r)
    w = _weights(s, rng)
    cap = ctx + r
    kc = np.zeros((hkv, cap, s.head_dim), np.float32)
    vc = np.zeros((hkv, cap, s.head_dim), np.float32)
    kc[:, :ctx] = rng.standard_normal((hkv, ctx, s.head_dim))
    vc[:, :ctx] = rng.standard_normal((hkv, ctx, s.head_dim))
    X = rng.standard_normal((2, r, s.d_model)).astype(np.float32)
    got = ko.attention_item_window(X, w["w_qkv"], w["w_o"], kc, vc, ctx, s)
    k, v = _kv_of_tokens(X, w, ctx, s)
    for m in range(2):
        kcm, vcm = kc.copy(), vc.copy()
        for t in range(r):
            # token t alone, with the cache holding positions 0 .. ctx+t-1
            one = ko.attention_item(X[m, t][None], w["w_qkv"], w["w_o"], kcm, vcm, ctx + t, s)
            assert np.allclose(got[m, t], one[0], rtol=2e-5, atol=2e-6), (m, t)
            kcm[:, ctx + t], vcm[:, ctx + t] = k[m, t], v[m, t]


def test_window_token_ignores_later_tokens():
    s = _shape()
    rng = np.random.default_rng(7)
    w = _weights(s, rng)
    kc = rng.standard_normal((2, 6, 8)).astype(np.float32)
    vc = rng.standard_normal((2, 6, 8)).astype(np.float32)
    X = rng.standard_normal((3, 4, s.d_model)).astype(np.float32)
    a = ko.attention_item_window(X, w["w_qkv"], w["w_o"], kc, vc, 6, s)
    Y = X.copy()
    Y[:, 3] = rng.standard_normal((3, s.d_model))
    b = ko.attention_item_window(Y, w["w_qkv"], w["w_o"], kc, vc, 6, s)
    assert np.array_equal(a[:, :3], b[:, :3])
    assert not np.allclose(a[:, 3], b[:, 3])


def test_window_of_one_token_is_the_single_token_item():
    s = _shape()
    rng = np.random.default_rng(9)
    w = _weights(s, rng)
    kc = rng.standard_normal((2, 5, 8)).astype(np.float32)
    vc = rng.standard_normal((2, 5, 8)).astype(np.float32)
    X = rng.standard_normal((4, s.d_model)).astype(np.float32)
    a = ko.attention_item(X, w["w_qkv"], w["w_o"], kc, vc, 5, s)
    b = ko.attention_item_window(X[:, None, :], w["w_qkv"], w["w_o"], kc, vc, 5, s)[:, 0]
    assert np.allclose(a, b, rtol=1e-5, atol=1e-6)


def test_frobenius_cosine_of_window_states():
    rng = np.random.default_rng(3)
    A = rng.standard_normal((5, 3, 7))
    ref = rng.standard_normal((3, 7))
    c = ko.cos_rows(A, ref)
    for m in range(5):
        want = float(np.sum(A[m] * ref)) / (np.linalg.norm(A[m]) * np.linalg.norm(ref))
        assert c[m] == pytest.approx(want, rel=1e-12)
    # r identical tokens: the same cosine as one token
    x = rng.standard_normal((4, 7))
    y = rng.standard_normal(7)
    assert np.allclose(ko.cos_rows(np.repeat(x[:, None], 3, axis=1), np.tile(y, (3, 1))),
                       ko.cos_rows(x, y))


def _small_window_problem(r, n_layers=4):
    wl = scaled(WORKLOADS["tiny"], n_layers=n_layers, name="win_t")
    layers = [synth.layer_weights(wl, l, 0) for l in range(n_layers)]
    kv = [synth.kv_cache(wl, l, 0, 64, 0) for l in range(n_layers)]
    x0 = synth.x0_window(wl, r, 0, 0, 0)
    items = ko.DecoderItems(decoder_shape(wl), layers, kv, 40, cache_widened=True)
    return wl, items, x0


@pytest.mark.parametrize("r", [2, 3])
def test_window_dp_against_enumeration(r):
    wl, items, x0 = _small_window_problem(r)
    n_items = 2 * wl.shape.n_layers
    t = ko.item_latencies(wl.shape.n_layers, 40, 1.0, 0.01, 2.0)
    w = ko.item_weights(t, 12)
    dp = ko.knapsack_dp(items, n_items, w, x0, 12)
    assert np.array_equal(dp.states[0], x0)          # budget 0: every item skipped
    ids, cos_all = ko.brute_force(items, n_items, x0)
    weight = np.array([sum(int(w[i]) for i in range(n_items) if (s >> i) & 1) for s in ids])
    for b in np.nonzero(dp.valid)[0]:
        # the kept set has weight b, and re-running it gives the DP's cosine
        assert int(np.sum(w[dp.bits[b]])) == b
        c = ko.eval_subsets(items, n_items, x0, dp.bits[b][None])[0]
        assert c == pytest.approx(dp.cos[b], abs=1e-6)
        assert dp.cos[b] <= np.max(cos_all[weight == b]) + 1e-6
    # the full set reproduces the reference
    full = np.ones((1, n_items), dtype=bool)
    assert ko.eval_subsets(items, n_items, x0, full)[0] == pytest.approx(1.0, abs=1e-12)


def test_greedy_tokens_is_argmax_of_normed_logits():
    rng = np.random.default_rng(5)
    X = rng.standard_normal((6, 5)).astype(np.float32)
    W = rng.standard_normal((7, 5)).astype(np.float32)
    tok, margin = ko.greedy_tokens(X, W, 1e-5)
    for m in range(6):
        x = X[m].astype(np.float64)
        xn = x / math.sqrt(float(np.mean(x * x)) + 1e-5)
        logits = [float(np.dot(xn, W[v].astype(np.float64))) for v in range(7)]
        best = max(range(7), key=lambda v: (logits[v], -v))
        assert tok[m] == best
        srt = sorted(logits)
        assert margin[m] == pytest.approx(srt[-1] - srt[-2], rel=1e-6)  # float32 RMSNorm


def test_alpha_lm_head_planted_tokens():
    d, r = 6, 4
    W = np.eye(d, dtype=np.float32)                   # token = largest coordinate
    ref = np.zeros((r, d), np.float32)
    for t in range(r):
        ref[t, t] = 1.0                               # full-model tokens 0, 1, 2, 3
    states = np.zeros((3, r, d), np.float32)
    states[0] = ref                                   # all four match
    states[1, :, 5] = 1.0                             # token 5 everywhere: no match
    states[2] = ref
    states[2, 1] = 0.0
    states[2, 1, 4] = 1.0                             # one of four replaced
    a = ko.alpha_lm_head(states, np.array([True, True, True]), ref, W, 1e-5)
    assert list(a) == [1.0, 0.0, 0.75]
    a = ko.alpha_lm_head(states, np.array([True, False, True]), ref, W, 1e-5)
    assert list(a) == [1.0, 0.0, 0.75]


def test_alpha_lm_head_on_window_dp_states():
    r = 3
    wl, items, x0 = _small_window_problem(r)
    n_items = 2 * wl.shape.n_layers
    t = ko.item_latencies(wl.shape.n_layers, 40, 1.0, 0.01, 2.0)
    w = ko.item_weights(t, 12)
    dp = ko.knapsack_dp(items, n_items, w, x0, 12)
    W = synth.lm_head(wl, vocab=64)
    a = ko.alpha_lm_head(dp.states, dp.valid, dp.ref, W, wl.shape.rms_eps)
    assert np.all(np.isin(np.round(a * r, 9), np.arange(r + 1)))
    assert np.all(a[~dp.valid] == 0.0)
    assert ko.alpha_lm_head(dp.ref[None], np.array([True]), dp.ref, W, 1e-5)[0] == 1.0

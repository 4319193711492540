"""Pins for the oracle's decoder item math (RMSNorm, RoPE, attention, SwiGLU MLP)."""
import math

import numpy as np
import pytest
from scipy.special import expit

from oracle import knapspec_oracle as ko


def _shape(**kw):
    base = dict(n_layers=1, d_model=32, n_q_heads=4, n_kv_heads=2, head_dim=8, d_ff=48,
                rms_eps=1e-5, rope_theta=1e4)
    base.update(kw)
    return ko.DecoderShape(**base)


def _weights(s, rng, sigma=0.2):
    q_dim = s.n_q_heads * s.head_dim
    return {
        "w_qkv": (rng.standard_normal(((s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim, s.d_model)) * sigma).astype(np.float32),
        "w_o": (rng.standard_normal((s.d_model, q_dim)) * sigma).astype(np.float32),
        "w_gate_up": (rng.standard_normal((2 * s.d_ff, s.d_model)) * sigma).astype(np.float32),
        "w_down": (rng.standard_normal((s.d_model, s.d_ff)) * sigma).astype(np.float32),
    }


def test_rmsnorm_definition():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64)).astype(np.float32) * 3
    y = ko.rmsnorm(x, 1e-5)
    ms = np.mean(x.astype(np.float64) ** 2, axis=1)
    # mean square of the output is ms / (ms + eps); direction unchanged
    assert np.allclose(np.mean(y.astype(np.float64) ** 2, axis=1), ms / (ms + 1e-5), rtol=1e-5)
    assert np.allclose(ko.cos_rows(y, x[0])[0], 1.0, atol=1e-6)


def test_rope_hand_value_and_properties():
    # dh = 2: a single pair rotated by angle pos * theta^0 = pos
    c, s = ko.rope_cos_sin(1, 2, 1e4)
    out = ko.rope(np.array([1.0, 0.0], np.float32), c, s)
    assert out == pytest.approx([math.cos(1.0), math.sin(1.0)], abs=1e-7)
    rng = np.random.default_rng(1)
    q = rng.standard_normal(128).astype(np.float32)
    k = rng.standard_normal(128).astype(np.float32)
    # position 0 is the identity; rotation preserves the norm
    c0, s0 = ko.rope_cos_sin(0, 128, 5e5)
    assert np.array_equal(ko.rope(q, c0, s0), q)
    for pos in (1, 17, 4096, 32768):
        cp, sp = ko.rope_cos_sin(pos, 128, 5e5)
        assert np.linalg.norm(ko.rope(q, cp, sp)) == pytest.approx(np.linalg.norm(q), rel=1e-5)
    # relative-position property: <R(m) q, R(n) k> depends on m - n only
    def dot(m, n):
        cm, sm = ko.rope_cos_sin(m, 128, 1e4)
        cn, sn = ko.rope_cos_sin(n, 128, 1e4)
        return float(np.dot(ko.rope(q, cm, sm).astype(np.float64), ko.rope(k, cn, sn)))
    assert dot(10, 3) == pytest.approx(dot(107, 100), rel=1e-4)
    # rotate-half pairing: element j pairs with j + dh/2 (not j+1)
    e = np.zeros(8, np.float32)
    e[1] = 1.0
    cp, sp = ko.rope_cos_sin(3, 8, 1e4)
    r = ko.rope(e, cp, sp)
    assert np.count_nonzero(np.abs(r) > 1e-9) == 2 and abs(r[5]) > 0


def _loop_attention(X, w, kc, vc, ctx, s):
    """Scalar-loop attention from the definition (softmax over ctx cached + 1 own position)."""
    X64 = X.astype(np.float64)
    M, d = X.shape
    hq, hkv, dh = s.n_q_heads, s.n_kv_heads, s.head_dim
    out = np.zeros((M, d))
    for r in range(M):
        x = X64[r]
        xn = x / math.sqrt(sum(v * v for v in x) / d + s.rms_eps)
        qkv = w["w_qkv"].astype(np.float64) @ xn
        o = np.zeros(hq * dh)
        half = dh // 2
        for h in range(hq):
            c = h * hkv // hq
            q = qkv[h * dh:(h + 1) * dh]
            k = qkv[(hq + c) * dh:(hq + c + 1) * dh]
            v = qkv[(hq + hkv + c) * dh:(hq + hkv + c + 1) * dh]
            def rot(z):
                y = np.empty(dh)
                for j in range(half):
                    a = ctx * s.rope_theta ** (-2.0 * j / dh)
                    y[j] = z[j] * math.cos(a) - z[j + half] * math.sin(a)
                    y[j + half] = z[j + half] * math.cos(a) + z[j] * math.sin(a)
                return y
            q, k = rot(q), rot(k)
            scores = [float(np.dot(q, kc[c, p].astype(np.float64))) / math.sqrt(dh) for p in range(ctx)]
            scores.append(float(np.dot(q, k)) / math.sqrt(dh))
            mx = max(scores)
            ex = [math.exp(z - mx) for z in scores]
            den = sum(ex)
            acc = np.zeros(dh)
            for p in range(ctx):
                acc += ex[p] / den * vc[c, p].astype(np.float64)
            acc += ex[-1] / den * v
            o[h * dh:(h + 1) * dh] = acc
        out[r] = x + w["w_o"].astype(np.float64) @ o
    return out


@pytest.mark.parametrize("hq,hkv,ctx", [(4, 2, 9), (4, 4, 5), (4, 1, 3), (2, 2, 0)])
def test_attention_matches_scalar_loops(hq, hkv, ctx):
    s = _shape(n_q_heads=hq, n_kv_heads=hkv)
    rng = np.random.default_rng(hq * 10 + hkv + ctx)
    w = _weights(s, rng)
    kc = rng.standard_normal((hkv, max(ctx, 1), s.head_dim)).astype(np.float32)
    vc = rng.standard_normal((hkv, max(ctx, 1), s.head_dim)).astype(np.float32)
    X = rng.standard_normal((3, s.d_model)).astype(np.float32)
    got = ko.attention_item(X, w["w_qkv"], w["w_o"], kc, vc, ctx, s)
    want = _loop_attention(X, w, kc, vc, ctx, s)
    assert np.allclose(got, want, rtol=1e-4, atol=1e-5)


def test_attention_without_cache_returns_own_value():
    s = _shape()
    rng = np.random.default_rng(3)
    w = _weights(s, rng)
    X = rng.standard_normal((4, s.d_model)).astype(np.float32)
    got = ko.attention_item(X, w["w_qkv"], w["w_o"], np.zeros((2, 1, 8), np.float32),
                            np.zeros((2, 1, 8), np.float32), 0, s)
    xn = X / np.sqrt(np.mean(X.astype(np.float64) ** 2, axis=1, keepdims=True) + 1e-5)
    v = xn @ w["w_qkv"][(4 + 2) * 8:].T.astype(np.float64)  # [M][hkv*dh]
    o = np.concatenate([v[:, (h // 2) * 8:(h // 2 + 1) * 8] for h in range(4)], axis=1)
    assert np.allclose(got, X + o @ w["w_o"].T, rtol=1e-5, atol=1e-6)


def test_gqa_equals_mha_with_duplicated_kv_heads():
    s_g = _shape(n_q_heads=4, n_kv_heads=2)
    s_m = _shape(n_q_heads=4, n_kv_heads=4)
    rng = np.random.default_rng(4)
    w = _weights(s_g, rng)
    dh, ctx = 8, 6
    kc = rng.standard_normal((2, ctx, dh)).astype(np.float32)
    vc = rng.standard_normal((2, ctx, dh)).astype(np.float32)
    qrows = w["w_qkv"][: 4 * dh]
    krows = w["w_qkv"][4 * dh: 6 * dh].reshape(2, dh, -1)
    vrows = w["w_qkv"][6 * dh:].reshape(2, dh, -1)
    dup = lambda a: np.repeat(a, 2, axis=0)
    w_m = dict(w)
    w_m["w_qkv"] = np.concatenate([qrows, dup(krows).reshape(4 * dh, -1),
                                   dup(vrows).reshape(4 * dh, -1)], axis=0)
    X = rng.standard_normal((3, s_g.d_model)).astype(np.float32)
    a = ko.attention_item(X, w["w_qkv"], w["w_o"], kc, vc, ctx, s_g)
    b = ko.attention_item(X, w_m["w_qkv"], w["w_o"], dup(kc), dup(vc), ctx, s_m)
    assert np.allclose(a, b, rtol=1e-5, atol=1e-6)


def test_mlp_swiglu_definition():
    s = _shape()
    rng = np.random.default_rng(5)
    w = _weights(s, rng)
    X = rng.standard_normal((4, s.d_model)).astype(np.float64)
    xn = X / np.sqrt(np.mean(X ** 2, axis=1, keepdims=True) + 1e-5)
    gu = xn @ w["w_gate_up"].T.astype(np.float64)
    g, u = gu[:, :48], gu[:, 48:]
    want = X + (g * expit(g) * u) @ w["w_down"].T.astype(np.float64)
    got = ko.mlp_item(X.astype(np.float32), w["w_gate_up"], w["w_down"], s)
    assert np.allclose(got, want, rtol=1e-5, atol=1e-5)


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F80], dtype=np.uint16)
    vals = ko.widen(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[3] == 0.0 and np.isinf(vals[4])
    assert vals[2] == pytest.approx(3.140625)

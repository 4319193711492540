"""Host-side checks of the C ABI (no GPU needed): exports, host-only entry points vs the
oracle, argument validation and error codes."""
import math
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import knapspec_oracle as ko
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "knapspec.h")


@pytest.fixture(scope="module")
def ks():
    lib = os.path.join(ROOT, "draft_layer_selection_amd", "libknapspec.so")
    if not os.path.exists(lib):
        from draft_layer_selection_amd import build

        build.build()
    from draft_layer_selection_amd import knapspec

    return knapspec


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(knapspec_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(ks):
    names = header_functions()
    assert len(names) == 17, names
    out = subprocess.run(["nm", "-D", "--defined-only", ks.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (knapspec_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(ks.lib, n)
    assert set(ks.SIGNATURES) == set(names)
    # nothing else leaks out of the library under the knapspec_ prefix
    assert exported == set(names)


def test_version_and_mask_words(ks):
    assert ks.knapspec_abi_version() == 3
    assert [ks.knapspec_mask_words(n) for n in (1, 8, 32, 33, 80)] == [1, 1, 1, 2, 3]


@pytest.mark.parametrize("name", ["tiny", "qwen3_1p7b_4k", "llama3_8b_32k", "llama3_70b_32k"])
def test_item_weights_match_oracle(ks, name):
    wl = WORKLOADS[name]
    s, lat = wl.shape, wl.latency
    for ctx in (0, 1, 255, wl.ctx, 2 * wl.ctx + 3):
        t, w = ks.item_weights(s.n_layers, ctx, wl.n_budgets, lat.attn_base, lat.attn_per_token,
                               lat.mlp, lat.fixed)
        t_o = ko.item_latencies(s.n_layers, ctx, lat.attn_base, lat.attn_per_token, lat.mlp)
        w_o = ko.item_weights(t_o, wl.n_budgets)
        assert np.array_equal(t, t_o)
        assert np.array_equal(w, w_o.astype(np.int32))


def test_item_weights_random_and_per_item(ks):
    rng = np.random.default_rng(0)
    for _ in range(200):
        L = int(rng.integers(1, 12))
        B = int(rng.integers(2, 300))
        per = rng.uniform(0, 10, size=2 * L)
        per[rng.random(2 * L) < 0.1] = 0.0
        if per.sum() == 0:
            per[0] = 1.0
        t, w = ks.item_weights(L, 17, B, 1.0, 0.1, 2.0, 0.0, per_item=per)
        w_o = ko.item_weights(per, B)
        assert np.array_equal(t, per) and np.array_equal(w, w_o.astype(np.int32))


def test_tpt_select_matches_oracle(ks):
    rng = np.random.default_rng(1)
    for trial in range(300):
        B = int(rng.integers(1, 40))
        alpha = rng.uniform(-0.2, 1.1, size=B).astype(np.float32)
        alpha[rng.random(B) < 0.1] = 1.0
        if trial % 7 == 0:
            alpha[:] = alpha[0]  # many exact ties
        t_d = rng.uniform(0, 5, size=B)
        valid = rng.random(B) < 0.8
        t_t = float(rng.uniform(1, 20))
        g0 = int(rng.integers(1, 6))
        g1 = g0 + int(rng.integers(0, 10))
        got = ks.tpt_select(alpha, t_d, valid, t_t, g0, g1)
        a64 = np.clip(alpha.astype(np.float64), 0, 1)
        want = ko.tpt_select(a64, t_d, valid, t_t, g0, g1)
        assert got[:2] == want[:2], (got, want)
        if want[0] >= 0:
            assert got[2] == pytest.approx(want[2], rel=1e-14)
        else:
            assert math.isnan(got[2])


def test_error_codes(ks):
    a = np.zeros(3, np.float32)
    with pytest.raises(ks.KnapSpecError) as e:
        ks.tpt_select(a, np.zeros(3), np.ones(3, bool), 1.0, 5, 2)
    assert e.value.code == ks.KNAPSPEC_EINVAL and "gamma" in str(e.value)
    with pytest.raises(ks.KnapSpecError) as e:
        ks.item_weights(4, 10, 32, -1.0, 0.0, 1.0)
    assert e.value.code == ks.KNAPSPEC_EINVAL
    with pytest.raises(ks.KnapSpecError) as e:
        ks.item_weights(4, 10, 1, 1.0, 0.0, 1.0)
    assert e.value.code == ks.KNAPSPEC_EINVAL
    with pytest.raises(ks.KnapSpecError) as e:
        ks.item_weights(2, 10, 32, 0.0, 0.0, 0.0)
    assert e.value.code == ks.KNAPSPEC_EINVAL and "positive" in str(e.value)


def _desc(ks, **kw):
    d = dict(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, d_ff=512,
             dtype=ks.KNAPSPEC_F32, rms_eps=1e-5, rope_theta=1e4, max_budgets=16, max_seqs=1,
             max_ctx=64)
    d.update(kw)
    return ks.knapspec_model_desc(**d)


def _load(ks, desc, null_weight=False):
    import ctypes as C

    arr = (ks.knapspec_layer_weights * desc.n_layers)()
    for i in range(desc.n_layers):
        p = 0 if (null_weight and i == 1) else 0x1000
        arr[i] = ks.knapspec_layer_weights(0x1000, 0x1000, p, 0x1000)
    h = C.c_void_p()
    rc = ks.knapspec_load_model(C.byref(desc), arr, None, C.byref(h))
    return rc, h


def test_load_model_validation(ks):
    bad = [dict(n_q_heads=3), dict(head_dim=63), dict(dtype=7), dict(max_budgets=1),
           dict(max_budgets=5000), dict(max_seqs=0), dict(max_ctx=-1), dict(rms_eps=0.0),
           dict(d_model=0), dict(max_window=-1), dict(max_window=ks.KNAPSPEC_WINDOW_MAX + 1)]
    for kw in bad:
        rc, _ = _load(ks, _desc(ks, **kw))
        assert rc == ks.KNAPSPEC_EINVAL, kw
        assert ks.knapspec_last_error().decode()
    rc, _ = _load(ks, _desc(ks), null_weight=True)
    assert rc == ks.KNAPSPEC_EINVAL and b"NULL" in ks.knapspec_last_error()
    rc, _ = _load(ks, _desc(ks, dtype=ks.KNAPSPEC_BF16, head_dim=96, n_q_heads=2, n_kv_heads=2))
    assert rc == ks.KNAPSPEC_EUNSUPPORTED


def test_load_model_alloc_failure_hook(ks, monkeypatch):
    monkeypatch.setenv("KNAPSPEC_TEST_FAIL_ALLOC", "1")
    rc, _ = _load(ks, _desc(ks))
    assert rc == ks.KNAPSPEC_ENOMEM


def test_load_model_without_device(ks):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc, _ = _load(ks, _desc(ks))
    assert rc == ks.KNAPSPEC_EHIP and b"device" in ks.knapspec_last_error()


def test_solve_rejects_null(ks):
    import ctypes as C

    rc = ks.knapspec_solve(None, None, None)
    assert rc == ks.KNAPSPEC_EINVAL
    ks.knapspec_free_model(None)  # no-op


def test_fit_latency_matches_least_squares(ks):
    """The host line fit against numpy's least-squares polynomial fit, on noisy and exact
    lines, and its R^2 against the definition 1 - RSS/TSS."""
    rng = np.random.default_rng(5)
    n = np.array([0, 1024, 4096, 8192, 16384, 32768], dtype=np.int32)
    for a0, b0, noise in ((10.0, 5e-4, 0.0), (37.7, 5.12e-4, 0.3), (3.1, 0.0, 0.05)):
        t = a0 + b0 * n + noise * rng.standard_normal(len(n))
        a, b, r2 = ks.fit_latency(n, t)
        bb, aa = np.polyfit(n.astype(np.float64), t, 1)
        assert a == pytest.approx(aa, rel=1e-9, abs=1e-9)
        assert b == pytest.approx(bb, rel=1e-9, abs=1e-15)
        resid = t - (aa + bb * n)
        tss = np.sum((t - t.mean()) ** 2)
        want = 1.0 - np.sum(resid ** 2) / tss if tss > 0 else 1.0
        assert r2 == pytest.approx(want, rel=1e-9, abs=1e-12)
    # exact line: R^2 = 1
    assert ks.fit_latency([1, 2, 3], [3.0, 5.0, 7.0]) == pytest.approx((1.0, 2.0, 1.0))


def test_fit_latency_rejects_bad_input(ks):
    with pytest.raises(ks.KnapSpecError):
        ks.fit_latency([5], [1.0])
    with pytest.raises(ks.KnapSpecError):
        ks.fit_latency([7, 7, 7], [1.0, 2.0, 3.0])
    with pytest.raises(ks.KnapSpecError):
        ks.fit_latency([1, 2], [1.0, float("nan")])


def test_profile_items_rejects_null_model(ks):
    import ctypes as C

    out = (C.c_double * 1)()
    mlp = C.c_double()
    n = (C.c_int32 * 1)(0)
    rc = ks.knapspec_profile_items(None, None, n, 1, 1, None, out, C.byref(mlp))
    assert rc == ks.KNAPSPEC_EINVAL


def test_set_lm_head_rejects_null_model(ks):
    assert ks.knapspec_set_lm_head(None, 0x1000, 64) == ks.KNAPSPEC_EINVAL
    assert b"NULL" in ks.knapspec_last_error()


def test_window_struct_layout(ks):
    import ctypes as C

    # the appended fields sit at the end of their C structs (ABI version 3)
    assert ks.knapspec_model_desc.max_window.offset == 12 * 4
    # ctx_len, ctx_capacity (int32), k_cache, v_cache, x0 (pointers), then window
    assert ks.knapspec_seq.window.offset == 8 + 3 * C.sizeof(C.c_void_p)
    assert ks.knapspec_result.tokens.offset == ks.knapspec_result.alpha.offset + C.sizeof(C.c_void_p)

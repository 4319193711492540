"""CPU checks of the test-side helpers the full-size parity tests rely on."""
import numpy as np

from oracle import knapspec_oracle as ko
from tests.helpers import LockstepSubsets, Problem, WidenedLayers, decoder_shape
from workloads import WORKLOADS, scaled


def test_lockstep_subsets_equal_eval_subsets_and_leave_the_dp_unchanged():
    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=3, d_model=256, n_q_heads=4,
                n_kv_heads=2, head_dim=64, d_ff=512, name="lockstep")
    p = Problem(wl, 0, ctxs=[70])
    lat = {"attn_base": wl.latency.attn_base, "attn_per_token": wl.latency.attn_per_token,
           "mlp": wl.latency.mlp, "fixed": 0.0}
    items = p.items(0)
    plain = ko.solve(decoder_shape(wl), None, None, p.x0[0], 70, lat, 24, (1, 8),
                     apply_item=items)
    n_items = 2 * wl.shape.n_layers
    rng = np.random.default_rng(0)
    bits = rng.random((9, n_items)) < 0.5
    bits[0] = False
    bits[1] = True
    lock = LockstepSubsets(items, p.x0[0], bits)
    got = ko.solve(decoder_shape(wl), None, None, p.x0[0], 70, lat, 24, (1, 8),
                   apply_item=lock)
    assert np.array_equal(got.dp.bits, plain.dp.bits)
    assert np.allclose(got.dp.cos[got.dp.valid], plain.dp.cos[plain.dp.valid], rtol=0, atol=1e-6)
    want = ko.eval_subsets(items, n_items, p.x0[0], bits)
    assert np.allclose(lock.cos(got.dp.ref), want, rtol=0, atol=1e-6)
    assert abs(lock.cos(got.dp.ref)[1] - 1.0) < 1e-6   # all items = the full model


def test_widened_layers_are_exact():
    wl = scaled(WORKLOADS["qwen3_1p7b_4k"], n_layers=2, d_model=128, n_q_heads=2,
                n_kv_heads=1, head_dim=64, d_ff=256)
    p = Problem(wl, 0, ctxs=[1])
    for keep in (False, True):
        wide = WidenedLayers(p.layers, threads=3, keep_all=keep)
        for l in (0, 1, 0):
            for k, v in p.layers[l].items():
                assert np.array_equal(wide[l][k], ko.widen(v))

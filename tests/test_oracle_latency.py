"""Pins for latencies and integer item weights (review, referee major comment 4)."""
import numpy as np
import pytest

from oracle import knapspec_oracle as ko
from workloads import WORKLOADS


def test_attention_latency_linear_mlp_flat():
    t1 = ko.item_latencies(4, 100, 2.0, 0.5, 7.0)
    t2 = ko.item_latencies(4, 300, 2.0, 0.5, 7.0)
    assert np.allclose(t1[0::2], 52.0) and np.allclose(t2[0::2], 152.0)
    assert np.allclose(t1[1::2], 7.0) and np.allclose(t2[1::2], 7.0)


def test_table_width_relation():
    # one weight per item type: K = sum(w) = (w_attn + w_mlp) * L
    for name, wl in WORKLOADS.items():
        if wl.n_seqs > 1:
            continue
        s, lat = wl.shape, wl.latency
        t = ko.item_latencies(s.n_layers, wl.ctx, lat.attn_base, lat.attn_per_token, lat.mlp)
        w = ko.item_weights(t, wl.n_budgets)
        assert len(set(w[0::2])) == 1 and len(set(w[1::2])) == 1
        assert int(w.sum()) == (int(w[0]) + int(w[1])) * s.n_layers


@pytest.mark.parametrize("name,wa,wm,total", [
    ("tiny", 2, 1, 24), ("qwen3_1p7b_4k", 2, 3, 140), ("llama3_8b_32k", 3, 5, 256),
    ("llama3_70b_32k", 1, 2, 240)])
def test_preset_weights(name, wa, wm, total):
    wl = WORKLOADS[name]
    s, lat = wl.shape, wl.latency
    t = ko.item_latencies(s.n_layers, wl.ctx, lat.attn_base, lat.attn_per_token, lat.mlp)
    # t_attn / Delta and t_mlp / Delta computed by hand for the tiny preset:
    # t_attn = 1 + 0.01*256 = 3.56, t_mlp = 2, Delta = 8*5.56/31 = 1.43484 -> 2.48 -> 2, 1.39 -> 1
    w = ko.item_weights(t, wl.n_budgets)
    assert (int(w[0]), int(w[1]), int(w.sum())) == (wa, wm, total)


def test_rounding_half_even_and_floor_one():
    # Delta = sum(t) / (B - 1) = 16 / 8 = 2: 3/2 = 1.5 -> 2 and 5/2 = 2.5 -> 2 (ties to even)
    assert list(ko.item_weights(np.array([3.0, 5.0, 8.0]), 9)) == [2, 2, 4]
    # Delta = 8 / 4 = 2: 0.5/2 = 0.25 rounds to 0 and is floored to 1; 1/2 = 0.5 -> 0 -> 1
    assert list(ko.item_weights(np.array([0.5, 1.0, 6.5]), 5)) == [1, 1, 3]
    # Delta = 6 / 4 = 1.5: 4.5/1.5 = 3, 0.75/1.5 = 0.5 -> 0 -> 1, 0.75 -> 1
    assert list(ko.item_weights(np.array([4.5, 0.75, 0.75]), 5)) == [3, 1, 1]

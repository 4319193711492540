"""Host-side tabulation of workloads.sweep on hand-made results (no GPU)."""
import types

import numpy as np

from workloads.sweep import _mask_bits, layer_set_stats


def test_mask_bits_decodes_items_across_words():
    masks = np.zeros((2, 2), dtype=np.uint64)
    masks[0, 0] = np.uint64((1 << 0) | (1 << 63))
    masks[1, 1] = np.uint64(1 << 5)  # item 69
    bits = _mask_bits(masks, 70)
    assert bits[0].nonzero()[0].tolist() == [0, 63]
    assert bits[1].nonzero()[0].tolist() == [69]


def test_layer_set_stats_counts_attention_and_mlp():
    # 3 layers = 6 items; budgets: 0 (nothing), 1 (attn 0 + mlp 0 + attn 2), 2 invalid
    masks = np.zeros((1, 3, 1), dtype=np.uint64)
    masks[0, 1, 0] = np.uint64(0b010011)
    res = types.SimpleNamespace(
        masks=masks, valid=np.array([[1, 1, 0]], dtype=np.uint8),
        best_budget=np.array([1], dtype=np.int32), best_gamma=np.array([4], dtype=np.int32),
        cos=np.array([[0.5, 0.9, np.nan]], dtype=np.float32))
    st = layer_set_stats(res, 0, 6)
    assert st["valid_budgets"] == 2
    assert (st["pick_budget"], st["pick_gamma"]) == (1, 4)
    assert (st["pick_attn_kept"], st["pick_mlp_kept"]) == (2, 1)
    assert st["mean_attn_kept_frac"] == (0 + 2) / 2 / 3
    assert st["mean_mlp_kept_frac"] == (0 + 1) / 2 / 3
    assert abs(st["pick_cos"] - 0.9) < 1e-7

"""Glue between the seeded workload generators and the oracle (test side only)."""
from __future__ import annotations

import numpy as np

from oracle import knapspec_oracle as ko
from workloads import synth
from workloads.configs import Workload


def decoder_shape(wl: Workload) -> ko.DecoderShape:
    s = wl.shape
    return ko.DecoderShape(s.n_layers, s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim,
                           s.d_ff, s.rms_eps, s.rope_theta)


class Problem:
    """Host copies of one workload's inputs (weights, caches, x0 per sequence)."""

    def __init__(self, wl: Workload, seed: int = 0, ctxs=None, cap=None):
        self.wl = wl
        self.seed = seed
        self.layers = [synth.layer_weights(wl, l, seed) for l in range(wl.shape.n_layers)]
        self.ctxs = list(ctxs) if ctxs is not None else synth.sequence_contexts(wl, seed)
        self.caps = [cap if cap is not None else max(c, 1) for c in self.ctxs]
        self.kv = [[synth.kv_cache(wl, l, q, self.caps[q], seed) for l in range(wl.shape.n_layers)]
                   for q in range(len(self.ctxs))]
        self.x0 = [synth.x0(wl, q, 0, seed) for q in range(len(self.ctxs))]

    def oracle(self, seq: int = 0, tau: float = -np.inf, skip_cap: int = -1,
               n_budgets=None, gamma=None, per_item=None, cache_widened=True):
        wl = self.wl
        lat = synth.latency_args(wl)
        return ko.solve(decoder_shape(wl), self.layers, self.kv[seq], self.x0[seq],
                        self.ctxs[seq], lat, n_budgets or wl.n_budgets, gamma or wl.gamma,
                        tau=tau, skip_cap=skip_cap, per_item=per_item,
                        cache_widened=cache_widened)

    def items(self, seq: int = 0, cache_widened=True) -> ko.DecoderItems:
        return ko.DecoderItems(decoder_shape(self.wl), self.layers, self.kv[seq],
                               self.ctxs[seq], cache_widened)

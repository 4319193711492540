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


class LockstepSubsets:
    """Item function for the oracle's DP that also carries a fixed list of item subsets
    through the same item calls, so one pass over the weights gives both the DP and the
    oracle's forward of each subset (rule P2's re-evaluation of the GPU's masks).

    At item i the DP's rows and the states of the subsets that execute item i are passed to
    ``items`` as one block; rows are independent in every item function, so each row's
    result is the item applied to that row.  ``cos(ref)`` gives the subsets' final cosines
    against the full model's state (the DP's reference row)."""

    def __init__(self, items, x0, bits: np.ndarray):
        self.items, self.bits = items, np.asarray(bits, dtype=bool)
        x0 = np.asarray(x0, dtype=np.float32)
        self.rows = np.repeat(x0[None], self.bits.shape[0], axis=0)

    def __call__(self, i: int, X: np.ndarray) -> np.ndarray:
        sel = np.nonzero(self.bits[:, i])[0]
        if len(sel) == 0:
            return self.items(i, X)
        out = self.items(i, np.concatenate([X, self.rows[sel]], axis=0))
        self.rows[sel] = out[len(X):]
        return out[: len(X)]

    def cos(self, ref: np.ndarray) -> np.ndarray:
        return ko.cos_rows(self.rows, ref)


class WidenedLayers:
    """Layer weights for the oracle, widened from bf16 bit patterns to float32 on demand by a
    thread pool (exact conversion, no arithmetic of the method).  With ``keep_all`` every
    widened layer is kept (shared by the oracle runs of several sequences); otherwise only the
    most recently used one, for decoders whose float32 weights do not fit in host memory."""

    def __init__(self, layers, threads: int = 16, keep_all: bool = False):
        from concurrent.futures import ThreadPoolExecutor

        self.layers, self._pool = layers, ThreadPoolExecutor(threads)
        self._threads = threads
        self._cur = (-1, None)
        self._all = {} if keep_all else None

    def __len__(self):
        return len(self.layers)

    def _widen(self, a: np.ndarray) -> np.ndarray:
        if a.dtype != np.uint16:
            return a
        out = np.empty(a.shape, dtype=np.float32)
        fa, fo = a.reshape(-1), out.reshape(-1)
        step = (fa.size + self._threads - 1) // self._threads

        def part(j):
            sl = slice(j * step, min(fa.size, (j + 1) * step))
            fo[sl] = (fa[sl].astype(np.uint32) << np.uint32(16)).view(np.float32)
        list(self._pool.map(part, range(self._threads)))
        return out

    def __getitem__(self, l: int):
        if self._all is not None:
            if l not in self._all:
                self._all[l] = {k: self._widen(v) for k, v in self.layers[l].items()}
            return self._all[l]
        if self._cur[0] != l:
            self._cur = (-1, None)
            self._cur = (l, {k: self._widen(v) for k, v in self.layers[l].items()})
        return self._cur[1]

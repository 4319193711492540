"""Upload a synthetic workload to the GPU and drive the library (harness side).

Weights, KV caches and x0 come from ``synth`` (seeded, host-generated) and are copied into
torch device tensors; the library receives only their device pointers.  Host copies can be
kept for the CPU oracle.  No part of the method's arithmetic lives here.
"""
from __future__ import annotations

import math
from typing import List, Optional

import numpy as np

from . import synth
from .configs import Workload


def _to_device(arr: np.ndarray, dtype: str, torch):
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to("cuda", non_blocking=False)


class DeviceProblem:
    """Device-resident inputs of one workload (all sequences at their initial context)."""

    def __init__(self, wl: Workload, seed: int = 0, ctxs: Optional[List[int]] = None,
                 caps: Optional[List[int]] = None, keep_host: bool = False,
                 max_budgets: Optional[int] = None, window: int = 1, lm_vocab: int = 0,
                 max_beam: int = 1):
        import torch

        from draft_layer_selection_amd import knapspec as ks

        self.torch, self.ks = torch, ks
        self.wl, self.seed = wl, seed
        s = wl.shape
        self.ctxs = list(ctxs) if ctxs is not None else synth.sequence_contexts(wl, seed)
        grow = wl.resolves * wl.tokens_per_resolve if wl.n_seqs > 1 else 0
        self.caps = list(caps) if caps is not None else [max(1, c + grow) for c in self.ctxs]
        self.host_layers = [] if keep_host else None
        self.host_kv = [[] for _ in self.ctxs] if keep_host else None
        self.layers = []
        for l in range(s.n_layers):
            hw = synth.layer_weights(wl, l, seed)
            self.layers.append({k: _to_device(v, s.dtype, torch) for k, v in hw.items()})
            if keep_host:
                self.host_layers.append(hw)
        self.k_cache = [[] for _ in self.ctxs]
        self.v_cache = [[] for _ in self.ctxs]
        for q, cap in enumerate(self.caps):
            for l in range(s.n_layers):
                k, v = synth.kv_cache(wl, l, q, cap, seed)
                self.k_cache[q].append(_to_device(k, s.dtype, torch))
                self.v_cache[q].append(_to_device(v, s.dtype, torch))
                if keep_host:
                    self.host_kv[q].append((k, v))
        # r-token window: x0 [r][d] per sequence (r = 1 keeps the single-token [d] layout)
        self.window = max(1, int(window))
        self.host_x0 = [synth.x0(wl, q, 0, seed) if self.window == 1
                        else synth.x0_window(wl, self.window, q, 0, seed)
                        for q in range(len(self.ctxs))]
        self.x0 = [torch.from_numpy(x).to("cuda") for x in self.host_x0]
        # inputs of the re-solve schedule (multi-sequence presets): x0 of every (seq, resolve),
        # resident on the device up front
        self.n_resolves = wl.resolves if wl.n_seqs > 1 else 1
        self.resolve_x0 = [[synth.x0(wl, q, r, seed) for r in range(self.n_resolves)]
                           for q in range(len(self.ctxs))]
        self.resolve_x0_dev = [[torch.from_numpy(x).to("cuda") for x in row]
                               for row in self.resolve_x0]
        desc = dict(n_layers=s.n_layers, d_model=s.d_model, n_q_heads=s.n_q_heads,
                    n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, d_ff=s.d_ff,
                    dtype=ks.KNAPSPEC_BF16 if s.dtype == "bf16" else ks.KNAPSPEC_F32,
                    rms_eps=s.rms_eps, rope_theta=s.rope_theta,
                    max_budgets=max_budgets or wl.n_budgets, max_seqs=len(self.ctxs),
                    max_ctx=max(self.caps), max_window=self.window, max_beam=max_beam)
        torch.cuda.synchronize()
        self.model = ks.Model(desc, self.layers)
        self._prepared = {}
        lat = wl.latency
        self.model.set_latency(lat.attn_base, lat.attn_per_token, lat.mlp, lat.fixed)
        # LM head of the acceptance estimate: host copy (widened) for the oracle, device copy
        # in the model dtype for the library
        self.lm_vocab = int(lm_vocab)
        self.host_lm = None
        if self.lm_vocab:
            self.host_lm = synth.lm_head(wl, self.lm_vocab, seed)
            raw = synth.lm_head(wl, self.lm_vocab, seed, bits=True)
            self.lm = _to_device(raw, s.dtype, torch)
            self.model.set_lm_head(self.lm, self.lm_vocab)

    def set_x0(self, q: int, x: np.ndarray):
        self.host_x0[q] = x
        self.x0[q].copy_(self.torch.from_numpy(x))

    def seq_args(self, ctxs: Optional[List[int]] = None, resolve: Optional[int] = None):
        """Arguments of one solve.  With ``resolve`` = r the sequences are at their r-th
        re-solve: context ctx0 + r * tokens_per_resolve and that re-solve's x0."""
        if resolve is not None:
            ctxs = self.resolve_ctxs(resolve)
        ctxs = ctxs if ctxs is not None else self.ctxs
        x0 = ([self.resolve_x0_dev[q][resolve] for q in range(len(ctxs))] if resolve is not None
              else self.x0)
        return [{"ctx": ctxs[q], "k_cache": self.k_cache[q], "v_cache": self.v_cache[q],
                 "x0": x0[q], "window": self.window} for q in range(len(ctxs))]

    def resolve_ctxs(self, r: int) -> List[int]:
        return [c + r * self.wl.tokens_per_resolve for c in self.ctxs]

    def solve(self, n_budgets=None, gamma=None, tau=-math.inf, max_skip_weight=-1, flags=0,
              ctxs=None, result=None, resolve=None, beam=1):
        wl = self.wl
        # the knapspec_seq array of a (contexts, re-solve) pair is built once: the tensors
        # behind it stay in place (set_x0 copies into them)
        key = (tuple(ctxs) if ctxs is not None else None, resolve)
        prep = self._prepared.get(key)
        if prep is None:
            prep = self._prepared[key] = self.model.prepare(self.seq_args(ctxs, resolve))
        return self.model.solve(prep, n_budgets or wl.n_budgets, gamma or wl.gamma, tau,
                                max_skip_weight, flags, result=result, beam=beam)

    def close(self):
        self.model.close()

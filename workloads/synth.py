"""Seeded synthetic inputs for the KnapSpec DP workloads.

Every tensor is a standard normal draw times sigma from numpy's PCG64, keyed by
``SeedSequence([seed, cfg_id, tensor_id, layer, seq, chunk])`` so that any slice can be
regenerated independently and in parallel.  Values are rounded to the model dtype:
float32 stays float32; bfloat16 is produced by round-to-nearest-even on the float32 bits
and returned as the raw uint16 bit pattern (numpy has no bfloat16 type).

Distributions (no values are printed on the pages; these are the recipe of this build):
  weights   N(0, 0.02^2)   row-major [out][in]: w_qkv [(hq+2hkv)*dh][d] (q|k|v blocks),
                           w_o [d][hq*dh], w_gate_up [2*ff][d] (gate|up blocks), w_down [d][ff]
  KV cache  N(0, 1)        [hkv][ctx][dh] per layer, treated as already position-rotated keys
  x0        N(0, 0.02^2)   the current token's input hidden state, [d]; for an r-token
                           window, [r][d] (token t of the window drawn under its own key)
  LM head   N(0, 0.02^2)   [vocab][d] (the cosine-margin lemma check and the acceptance
                           estimate over a window)

This module is shared by the GPU path's harness and by the CPU oracle's tests.  It holds
no part of the method's arithmetic: only random draws, dtype rounding and bookkeeping.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

from .configs import Workload

T_WQKV, T_WO, T_WGU, T_WDOWN, T_KCACHE, T_VCACHE, T_X0, T_CTX, T_LMHEAD, T_X0WIN = range(10)
CHUNK = 1 << 22

W_SIGMA = 0.02
KV_SIGMA = 1.0
X0_SIGMA = 0.02

_POOL: Optional[ThreadPoolExecutor] = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        n = max(1, min(16, len(os.sched_getaffinity(0))))
        _POOL = ThreadPoolExecutor(n)
    return _POOL


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (for harness-side conversions)."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _fill_chunk(out: np.ndarray, start: int, stop: int, key, sigma: float, bf16: bool) -> None:
    gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))
    vals = gen.standard_normal(stop - start, dtype=np.float32)
    if sigma != 1.0:
        vals *= np.float32(sigma)
    out[start:stop] = f32_to_bf16_bits(vals) if bf16 else vals


def normal(shape, sigma: float, dtype: str, key) -> np.ndarray:
    """Seeded N(0, sigma^2) draw of ``shape`` rounded to ``dtype`` ("f32" or "bf16" bits)."""
    n = int(np.prod(shape))
    bf16 = dtype == "bf16"
    flat = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    n_chunks = max(1, math.ceil(n / CHUNK))
    jobs = []
    for c in range(n_chunks):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        jobs.append((flat, lo, hi, list(key) + [c], sigma, bf16))
    if n_chunks == 1:
        _fill_chunk(*jobs[0])
    else:
        list(_pool().map(lambda a: _fill_chunk(*a), jobs))
    return flat.reshape(shape)


def layer_weights(wl: Workload, layer: int, seed: int = 0) -> Dict[str, np.ndarray]:
    s = wl.shape
    q_dim = s.n_q_heads * s.head_dim
    base = [seed, wl.cfg_id]
    return {
        "w_qkv": normal((s.qkv_rows, s.d_model), W_SIGMA, s.dtype, base + [T_WQKV, layer, 0]),
        "w_o": normal((s.d_model, q_dim), W_SIGMA, s.dtype, base + [T_WO, layer, 0]),
        "w_gate_up": normal((2 * s.d_ff, s.d_model), W_SIGMA, s.dtype, base + [T_WGU, layer, 0]),
        "w_down": normal((s.d_model, s.d_ff), W_SIGMA, s.dtype, base + [T_WDOWN, layer, 0]),
    }


def kv_cache(wl: Workload, layer: int, seq: int, ctx_cap: int, seed: int = 0):
    """K and V cache of one layer of one sequence: two arrays [hkv][ctx_cap][dh].

    Position p of the cache depends only on (seed, cfg, layer, seq, p // CHUNK-rows), so a
    longer capacity extends a shorter one with the same leading positions only when the
    per-head row count is unchanged; callers allocate the final capacity once.
    """
    s = wl.shape
    shape = (s.n_kv_heads, ctx_cap, s.head_dim)
    base = [seed, wl.cfg_id]
    k = normal(shape, KV_SIGMA, s.dtype, base + [T_KCACHE, layer, seq])
    v = normal(shape, KV_SIGMA, s.dtype, base + [T_VCACHE, layer, seq])
    return k, v


def x0(wl: Workload, seq: int = 0, resolve: int = 0, seed: int = 0) -> np.ndarray:
    """The current token's input state [d] in the model dtype, widened to float32."""
    s = wl.shape
    v = normal((s.d_model,), X0_SIGMA, s.dtype, [seed, wl.cfg_id, T_X0, resolve, seq])
    return bf16_bits_to_f32(v) if s.dtype == "bf16" else v


def x0_window(wl: Workload, r: int, seq: int = 0, resolve: int = 0, seed: int = 0) -> np.ndarray:
    """Input states [r][d] of an r-token window (model dtype, widened to float32).  r = 1
    gives x0() as a [1][d] array."""
    if r == 1:
        return x0(wl, seq, resolve, seed)[None, :]
    s = wl.shape
    v = normal((r, s.d_model), X0_SIGMA, s.dtype, [seed, wl.cfg_id, T_X0WIN, resolve, seq])
    return bf16_bits_to_f32(v) if s.dtype == "bf16" else v


def lm_head(wl: Workload, vocab: int = 4096, seed: int = 0, bits: bool = False) -> np.ndarray:
    """LM head [vocab][d]; model dtype widened to float32, or the raw bf16 bit patterns."""
    s = wl.shape
    v = normal((vocab, s.d_model), W_SIGMA, s.dtype, [seed, wl.cfg_id, T_LMHEAD, 0, 0])
    if bits:
        return v
    return bf16_bits_to_f32(v) if s.dtype == "bf16" else v


def sequence_contexts(wl: Workload, seed: int = 0) -> List[int]:
    """Initial context length of each sequence of a multi-sequence preset.

    Lognormal centred geometrically in [lo, hi]: ln n ~ N(ln(sqrt(lo*hi)), (ln(hi/lo)/4)^2),
    redrawn until lo <= n <= hi - resolves * tokens_per_resolve, so the cache never grows
    past hi.  Single-sequence presets return [wl.ctx].
    """
    if wl.ctx_range is None:
        return [wl.ctx] * wl.n_seqs
    lo, hi = wl.ctx_range
    top = hi - wl.resolves * wl.tokens_per_resolve
    gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wl.cfg_id, T_CTX])))
    mu = math.log(math.sqrt(lo * hi))
    sd = math.log(hi / lo) / 4.0
    out = []
    while len(out) < wl.n_seqs:
        n = int(round(math.exp(gen.normal(mu, sd))))
        if lo <= n <= top:
            out.append(n)
    return out


def latency_args(wl: Workload) -> dict:
    lat = wl.latency
    return {"attn_base": lat.attn_base, "attn_per_token": lat.attn_per_token,
            "mlp": lat.mlp, "fixed": lat.fixed}

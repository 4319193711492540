"""Synthetic workload presets for the KnapSpec layer-selection DP.

Five decoder shapes stand in for the Qwen3 / Llama-3 models the KnapSpec paper evaluates
("KnapSpec: Self-Speculative Decoding via Adaptive Layer Selection as a Knapsack Problem",
pith.science review, section "The reading", and the abstract: Qwen3 and Llama3 models of
1B to 70B parameters).  Only the shapes
are taken; weights, KV caches and inputs are seeded synthetic draws (see ``synth``).

Latency model.  The paper profiles one latency per Attention item (growing linearly with
the context length n) and one per MLP item (flat in n) on the machine it runs on, and the
review's list of free parameters records that these values are not reported.
For the four model-shaped presets we take the plainest stand-in: bandwidth-bound decode time
at 8 TB/s, i.e. t_attn(n) = (attention weight bytes + K/V bytes per cached token * n) / BW and
t_mlp = MLP weight bytes / BW, in microseconds, with no fixed overhead.  The tiny preset uses
the abstract units t_attn = 1 + 0.01 n, t_mlp = 2 given with it.

This module holds shapes and numbers only; it contains none of the method's arithmetic.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

HBM_BYTES_PER_US = 8.0e12 / 1.0e6  # 8 TB/s expressed in bytes per microsecond


@dataclasses.dataclass(frozen=True)
class LatencyModel:
    """t_attn(n) = attn_base + attn_per_token * n ; t_mlp flat ; fixed = per-pass overhead."""

    attn_base: float
    attn_per_token: float
    mlp: float
    fixed: float = 0.0


@dataclasses.dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    dtype: str  # "f32" or "bf16" (weights and KV cache)
    rms_eps: float = 1e-5
    rope_theta: float = 1e4

    @property
    def n_items(self) -> int:
        return 2 * self.n_layers

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def attn_weight_bytes(self) -> int:
        q_dim = self.n_q_heads * self.head_dim
        return (self.qkv_rows * self.d_model + self.d_model * q_dim) * self.elem_bytes

    def mlp_weight_bytes(self) -> int:
        return 3 * self.d_model * self.d_ff * self.elem_bytes

    def kv_bytes_per_token(self) -> int:
        """K and V bytes one cached position costs one layer."""
        return 2 * self.n_kv_heads * self.head_dim * self.elem_bytes


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    shape: ModelShape
    latency: LatencyModel
    ctx: int  # context length n for single-sequence presets
    n_budgets: int
    gamma: Tuple[int, int]
    n_seqs: int = 1
    # multi-sequence re-solve schedule (the 16-sequence preset only)
    resolves: int = 1
    tokens_per_resolve: int = 0
    ctx_range: Optional[Tuple[int, int]] = None


def bandwidth_latency(shape: ModelShape) -> LatencyModel:
    """Bandwidth-bound stand-in latencies in microseconds at 8 TB/s (see module docstring)."""
    return LatencyModel(
        attn_base=shape.attn_weight_bytes() / HBM_BYTES_PER_US,
        attn_per_token=shape.kv_bytes_per_token() / HBM_BYTES_PER_US,
        mlp=shape.mlp_weight_bytes() / HBM_BYTES_PER_US,
        fixed=0.0,
    )


TINY_SHAPE = ModelShape(8, 256, 4, 4, 64, 768, "f32", 1e-5, 1e4)
QWEN3_1P7B_SHAPE = ModelShape(28, 2048, 16, 8, 128, 6144, "bf16", 1e-5, 1e6)
LLAMA3_8B_SHAPE = ModelShape(32, 4096, 32, 8, 128, 14336, "bf16", 1e-5, 5e5)
LLAMA3_70B_SHAPE = ModelShape(80, 8192, 64, 8, 128, 28672, "bf16", 1e-5, 5e5)

WORKLOADS = {
    "tiny": Workload("tiny", 0, TINY_SHAPE, LatencyModel(1.0, 0.01, 2.0, 0.0), 256, 32, (1, 8)),
    "qwen3_1p7b_4k": Workload("qwen3_1p7b_4k", 1, QWEN3_1P7B_SHAPE,
                              bandwidth_latency(QWEN3_1P7B_SHAPE), 4096, 128, (1, 8)),
    "llama3_8b_32k": Workload("llama3_8b_32k", 2, LLAMA3_8B_SHAPE,
                              bandwidth_latency(LLAMA3_8B_SHAPE), 32768, 256, (1, 12)),
    "llama3_8b_x16": Workload("llama3_8b_x16", 3, LLAMA3_8B_SHAPE,
                              bandwidth_latency(LLAMA3_8B_SHAPE), 0, 256, (1, 12),
                              n_seqs=16, resolves=8, tokens_per_resolve=256,
                              ctx_range=(2048, 32768)),
    "llama3_70b_32k": Workload("llama3_70b_32k", 4, LLAMA3_70B_SHAPE,
                               bandwidth_latency(LLAMA3_70B_SHAPE), 32768, 256, (1, 12)),
}


def scaled(workload: Workload, **overrides) -> Workload:
    """A copy of a preset with some fields replaced (small parity cases)."""
    shape_keys = {f.name for f in dataclasses.fields(ModelShape)}
    shape_over = {k: v for k, v in overrides.items() if k in shape_keys}
    wl_over = {k: v for k, v in overrides.items() if k not in shape_keys}
    shape = dataclasses.replace(workload.shape, **shape_over) if shape_over else workload.shape
    return dataclasses.replace(workload, shape=shape, **wl_over)


def mask_words(n_layers: int) -> int:
    return int(math.ceil(2 * n_layers / 64))

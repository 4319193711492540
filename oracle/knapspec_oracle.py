"""CPU oracle of KnapSpec's layer-selection knapsack DP and Tokens-per-Time pick.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain reference that the GPU library
is checked against.  Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import it.  It shares no code with the HIP library and imports nothing from it.

Source: "KnapSpec: Self-Speculative Decoding via Adaptive Layer Selection as a Knapsack
Problem" (Cha, Kim, Han, Yang, Han), as described on the pith.science review page of
arXiv 2602.20217.  The page does not print Eq. (4)-(9) or Algorithms 1-2 in full; each
function below names the part of the page it follows and the reading taken where the page
is silent.  Precision: item math in float32 (bf16 weights and caches are widened exactly),
cosines and the TPT objective in float64.

Pins (tests that tie this code to something other than itself):
  * tpt_value / tpt_select      closed form vs explicit geometric sums, the alpha->0 and
                                alpha->1 limits, hand-derived values in tests/golden/.
  * knapsack_dp                 additive-orthogonal items reduce the DP to a textbook
                                exact-weight 0/1 knapsack; the paper's skipped-weight index
                                convention gives the same candidate sets; brute force over
                                all 2^16 subsets of the tiny decoder (gap reported).
  * item math                   RMSNorm definition, RoPE norm preservation and relative-
                                position property, attention special cases (no cache ->
                                own value; constant keys -> mean), loop-based attention on
                                tiny inputs, SwiGLU via scipy's logistic function.
  * item_latencies / weights    the table-size relation K = (w_attn + w_mlp) L and the
                                linear-in-context attention latency.
  * Lemma 4.1                   cosine-margin => same greedy token, on DP states and on
                                constructed pairs at the bound.
  * window (r > 1) attention    processing r tokens as one causal block equals decoding them
                                one at a time with each token's key/value appended to the
                                cache; a token never depends on later window tokens;
                                loop-based attention on tiny inputs.
  * alpha_lm_head               the full-model state scores 1; planted LM heads with known
                                greedy tokens; values on the grid {0, 1/r, ..., 1}.
  * knapsack_dp_beam            beam 1 is knapsack_dp exactly; a beam at least as wide as the
                                number of subsets of any weight is exhaustive enumeration
                                (the best subset per budget, brute force on small decoders).
  * draft_verify                with every item executed the draft is the target model, so the
                                verification accepts every draft token; the verification block
                                equals token-by-token decoding (window pin above).
Parity unpinned: the full DP at the Qwen3-1.7B, Llama-3-8B and Llama-3-70B shapes has no
independent check beyond the pins above and the per-mask self-consistency of the results.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

F32 = np.float32
F64 = np.float64


# --------------------------------------------------------------------------------------
# Latencies and integer item weights
# --------------------------------------------------------------------------------------

def item_latencies(n_layers: int, ctx: int, attn_base: float, attn_per_token: float,
                   mlp: float, per_item: Optional[Sequence[float]] = None) -> np.ndarray:
    """Per-item latency t_i for items 0..2L-1 (item 2l = Attention of layer l, 2l+1 = MLP).

    Review, "The reading": Attention latency grows linearly with the context length and
    MLP latency is flat.  ``per_item`` replaces the linear model when given.
    """
    if per_item is not None:
        t = np.asarray(per_item, dtype=F64).copy()
        assert t.shape == (2 * n_layers,)
        return t
    t = np.empty(2 * n_layers, dtype=F64)
    t[0::2] = attn_base + attn_per_token * float(ctx)
    t[1::2] = mlp
    return t


def item_weights(t: np.ndarray, n_budgets: int) -> np.ndarray:
    """Integer knapsack weights w_i from latencies.

    Review, referee major comment 4 (Section 3.6): weights are latencies divided by a
    quantum, w = t / Delta, and the DP table has K + 1 budget columns.  Reading taken here:
    the B budget columns span the full-model latency, Delta = sum(t) / (B - 1); each weight
    is t_i / Delta rounded half-to-even, with a floor of 1 so that no item is free.
    """
    assert n_budgets >= 2
    total = float(np.sum(t))
    assert total > 0.0
    delta = total / (n_budgets - 1)
    return np.maximum(1, np.rint(np.asarray(t, dtype=F64) / delta)).astype(np.int64)


# --------------------------------------------------------------------------------------
# Decoder item math (Llama-style pre-norm block; float32)
# --------------------------------------------------------------------------------------

def widen(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or float32 values -> float32 values (exact)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(F32)
    return np.asarray(a, dtype=F32)


def rmsnorm(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) over the last axis, unit gain."""
    x = x.astype(F32, copy=False)
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=F32)
    return x / np.sqrt(ms + F32(eps))


def rope_cos_sin(pos: int, head_dim: int, theta: float):
    """Rotation table at one position: angle_j = pos * theta^(-2j/dh), j < dh/2 (float64)."""
    j = np.arange(head_dim // 2, dtype=F64)
    ang = float(pos) * np.power(float(theta), -2.0 * j / head_dim)
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half rotary embedding of the last axis: pairs (j, j + dh/2)."""
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1).astype(F32)


def silu(z: np.ndarray) -> np.ndarray:
    return (z / (F32(1.0) + np.exp(-z))).astype(F32)


@dataclasses.dataclass
class DecoderShape:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    rms_eps: float = 1e-5
    rope_theta: float = 1e4


def attention_item(X: np.ndarray, w_qkv: np.ndarray, w_o: np.ndarray, k_cache: np.ndarray,
                   v_cache: np.ndarray, ctx: int, s: DecoderShape) -> np.ndarray:
    """One Attention item applied to every row of X [M][d] (the new token at position ctx).

    Each row is its own candidate hidden state; all rows share the cached keys/values of
    positions 0..ctx-1 (already rotated) and each row also attends to its own key/value at
    position ctx.  Query head h reads KV head h // (hq / hkv).  Returns X + o W_o^T.
    """
    M = X.shape[0]
    hq, hkv, dh = s.n_q_heads, s.n_kv_heads, s.head_dim
    G = hq // hkv
    xn = rmsnorm(X, s.rms_eps)
    qkv = xn @ w_qkv.T
    q = qkv[:, : hq * dh].reshape(M, hq, dh)
    k = qkv[:, hq * dh:(hq + hkv) * dh].reshape(M, hkv, dh)
    v = qkv[:, (hq + hkv) * dh:].reshape(M, hkv, dh)
    cos, sin = rope_cos_sin(ctx, dh, s.rope_theta)
    q = rope(q, cos, sin)
    k = rope(k, cos, sin)
    scale = F32(1.0 / np.sqrt(dh))
    o = np.empty((M, hq, dh), dtype=F32)
    for c in range(hkv):
        Q = q[:, c * G:(c + 1) * G, :].reshape(M * G, dh)
        s_self = np.sum(Q * np.repeat(k[:, c, :], G, axis=0), axis=1, dtype=F32) * scale
        v_self = np.repeat(v[:, c, :], G, axis=0)
        if ctx > 0:
            Kc = widen(k_cache[c, :ctx, :])
            Vc = widen(v_cache[c, :ctx, :])
            sc = (Q @ Kc.T) * scale
            mx = np.maximum(sc.max(axis=1), s_self)
            p = np.exp(sc - mx[:, None])
            p_self = np.exp(s_self - mx)
            den = p.sum(axis=1, dtype=F32) + p_self
            out = (p @ Vc + p_self[:, None] * v_self) / den[:, None]
        else:
            out = v_self
        o[:, c * G:(c + 1) * G, :] = out.reshape(M, G, dh)
    return (X + o.reshape(M, hq * dh) @ w_o.T).astype(F32)


def attention_item_window(X: np.ndarray, w_qkv: np.ndarray, w_o: np.ndarray,
                          k_cache: np.ndarray, v_cache: np.ndarray, ctx: int,
                          s: DecoderShape) -> np.ndarray:
    """One Attention item applied to r-token states X [M][r][d].

    Review, referee major comment 4: the DP table holds r x d hidden states per cell, r being
    the tokens of the recent-token cache (window m, free parameters).  Reading taken here:
    the r tokens of a state enter the item together as the newest positions ctx .. ctx+r-1
    (token t at position ctx + t); every token attends to the cached positions 0..ctx-1 and,
    causally, to the keys/values that the item computes for tokens 0..t of the same state.
    With r = 1 this is attention_item.
    """
    M, r, d = X.shape
    hq, hkv, dh = s.n_q_heads, s.n_kv_heads, s.head_dim
    G = hq // hkv
    xn = rmsnorm(X, s.rms_eps)
    qkv = xn @ w_qkv.T
    q = qkv[:, :, : hq * dh].reshape(M, r, hq, dh)
    k = qkv[:, :, hq * dh:(hq + hkv) * dh].reshape(M, r, hkv, dh)
    v = qkv[:, :, (hq + hkv) * dh:].reshape(M, r, hkv, dh)
    for t in range(r):
        cos, sin = rope_cos_sin(ctx + t, dh, s.rope_theta)
        q[:, t] = rope(q[:, t], cos, sin)
        k[:, t] = rope(k[:, t], cos, sin)
    scale = F32(1.0 / np.sqrt(dh))
    causal = np.tril(np.ones((r, r), dtype=bool))          # [t][t'] key t' visible to t
    o = np.empty((M, r, hq, dh), dtype=F32)
    for c in range(hkv):
        Q = q[:, :, c * G:(c + 1) * G, :]                    # [M][r][G][dh]
        Kw, Vw = k[:, :, c, :], v[:, :, c, :]                # [M][r'][dh]
        sw = np.einsum("mtgd,mud->mtgu", Q, Kw).astype(F32) * scale
        sw = np.where(causal[None, :, None, :], sw, -np.inf).astype(F32)
        mx = sw.max(axis=3)
        if ctx > 0:
            Kc = widen(k_cache[c, :ctx, :])
            Vc = widen(v_cache[c, :ctx, :])
            sc = (Q.reshape(M * r * G, dh) @ Kc.T).reshape(M, r, G, ctx) * scale
            mx = np.maximum(mx, sc.max(axis=3))
            pc = np.exp(sc - mx[..., None])
            num = (pc.reshape(-1, ctx) @ Vc).reshape(M, r, G, dh)
            den = pc.sum(axis=3, dtype=F32)
        else:
            num = np.zeros((M, r, G, dh), dtype=F32)
            den = np.zeros((M, r, G), dtype=F32)
        pw = np.exp(sw - mx[..., None]).astype(F32)           # masked keys give exp(-inf) = 0
        num = num + np.einsum("mtgu,mud->mtgd", pw, Vw).astype(F32)
        den = den + pw.sum(axis=3, dtype=F32)
        o[:, :, c * G:(c + 1) * G, :] = num / den[..., None]
    return (X + o.reshape(M, r, hq * dh) @ w_o.T).astype(F32)


def mlp_item(X: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray,
             s: DecoderShape) -> np.ndarray:
    """One MLP item: X + (silu(xn W_g^T) * (xn W_u^T)) W_d^T, rows independent."""
    xn = rmsnorm(X, s.rms_eps)
    gu = xn @ w_gate_up.T
    h = silu(gu[:, : s.d_ff]) * gu[:, s.d_ff:]
    return (X + h @ w_down.T).astype(F32)


class DecoderItems:
    """Item function F_i for one sequence: item 2l = Attention of layer l, 2l+1 = MLP.

    ``layers`` is a list of dicts with w_qkv, w_o, w_gate_up, w_down (float32 arrays or
    bf16 bit patterns); ``kv`` a list of (k_cache, v_cache) per layer, [hkv][cap][dh].
    """

    def __init__(self, shape: DecoderShape, layers: List[Dict[str, np.ndarray]],
                 kv: List, ctx: int, cache_widened: bool = False):
        self.s, self.layers, self.kv, self.ctx = shape, layers, kv, ctx
        self.cache_widened = cache_widened
        self._w: Dict[int, Dict[str, np.ndarray]] = {}

    def _weights(self, layer: int) -> Dict[str, np.ndarray]:
        if layer in self._w:
            return self._w[layer]
        w = {k: widen(v) for k, v in self.layers[layer].items()}
        if self.cache_widened:
            self._w[layer] = w
        return w

    def __call__(self, i: int, X: np.ndarray) -> np.ndarray:
        """X: [M][d] single-token states, or [M][r][d] r-token states (window)."""
        layer = i // 2
        w = self._weights(layer)
        if i % 2 == 0:
            kc, vc = self.kv[layer]
            if X.ndim == 3:
                return attention_item_window(X, w["w_qkv"], w["w_o"], kc, vc, self.ctx, self.s)
            return attention_item(X, w["w_qkv"], w["w_o"], kc, vc, self.ctx, self.s)
        if X.ndim == 3:
            M, r, d = X.shape
            return mlp_item(X.reshape(M * r, d), w["w_gate_up"], w["w_down"],
                            self.s).reshape(M, r, d)
        return mlp_item(X, w["w_gate_up"], w["w_down"], self.s)


# --------------------------------------------------------------------------------------
# The knapsack DP over items x budgets
# --------------------------------------------------------------------------------------

def cos_rows(A: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Cosine of each state A[m] with the state r, in float64; 0/0 gives NaN.

    An r-token state [r][d] is compared as the flattened r*d vector (the Frobenius inner
    product of the two matrices over the product of their Frobenius norms) -- the reading
    taken for the cosine of the paper's r x d states.
    """
    A64 = A.astype(F64).reshape(A.shape[0], -1)
    r64 = r.astype(F64).reshape(-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        return (A64 @ r64) / (np.sqrt(np.sum(A64 * A64, axis=1)) * np.sqrt(r64 @ r64))


@dataclasses.dataclass
class DPResult:
    bits: np.ndarray        # bool [B][n_items], True = item executed
    valid: np.ndarray       # bool [B]
    cos: np.ndarray         # float64 [B], NaN where invalid
    decisions: np.ndarray   # uint8 [n_items][B]: 0 skip, 1 execute, 255 invalid
    margins: np.ndarray     # float64 [n_items][B]: |c_e - c_s|, inf if one option, NaN if none
    states: np.ndarray      # float32 [B][d] (or [B][r][d]) final candidate states
    ref: np.ndarray         # float32 [d] (or [r][d]) full-model state after the last item


def knapsack_dp(apply_item: Callable[[int, np.ndarray], np.ndarray], n_items: int,
                w: Sequence[int], x0: np.ndarray, n_budgets: int, tau: float = -np.inf,
                skip_cap: int = -1) -> DPResult:
    """KnapSpec's parallel DP, one hidden state per (item, budget) cell.

    Review, "What carries the argument" and referee major comment 1 (Section 3.4, Eq. 8,
    Algorithm 1): one candidate state is kept per item and budget; at each item, for every
    budget, execute and skip are compared by cosine similarity to the full model's hidden
    state at the same depth, and the higher one is kept.  Referee minor comment 2 (Eq. 7 vs
    Algorithm 1) shows that the paper indexes budgets by skipped weight; here budget b is the
    used weight sum_{executed} w_i, which maps onto the skipped index j by b = P_i - j with
    P_i = w_0 + ... + w_i (the tests check the two give identical candidate sets).

    Readings where the page is silent:
      * Initialisation: budget 0 holds x0 with the empty set; other budgets start empty.
      * The full-model reference is the same input pushed through every item.
      * Execute candidate at b comes from b - w_i; skip candidate is the state already at b;
        both are compared against the reference after item i.  Budgets above B - 1 are
        not kept.
      * Exact ties keep skip (minor comment 4 leaves tie handling open).  A NaN cosine counts
        as minus infinity.
      * Pruning (free parameter tau, Figure 4 caption): a kept cosine below tau makes the
        cell invalid.  ``skip_cap`` >= 0 invalidates cells whose skipped weight P_i - b
        exceeds it (the review's editorial reading of a K/2 skip cap).
    """
    B = int(n_budgets)
    x0 = np.asarray(x0, dtype=F32)           # [d], or [r][d] for r-token states
    g = np.zeros((B,) + x0.shape, dtype=F32)
    valid = np.zeros(B, dtype=bool)
    bits = np.zeros((B, n_items), dtype=bool)
    g[0] = x0
    valid[0] = True
    ref = x0.copy()
    decisions = np.full((n_items, B), 255, dtype=np.uint8)
    margins = np.full((n_items, B), np.nan, dtype=F64)
    kept = np.full(B, np.nan, dtype=F64)
    prefix = 0
    budgets = np.arange(B)
    for i in range(n_items):
        wi = int(w[i])
        prefix += wi
        src = np.nonzero(valid[: max(0, B - wi)])[0]
        rows = np.concatenate([g[src], ref[None]], axis=0)
        out = apply_item(i, rows)
        ex, ref_new = out[:-1], out[-1].astype(F32)
        tgt = src + wi

        c_exec = np.full(B, -np.inf)
        c_skip = np.full(B, -np.inf)
        if len(src):
            c_exec[tgt] = cos_rows(ex, ref_new)
        if valid.any():
            c_skip[valid] = cos_rows(g[valid], ref_new)
        c_exec[np.isnan(c_exec)] = -np.inf
        c_skip[np.isnan(c_skip)] = -np.inf

        take = c_exec > c_skip
        best = np.where(take, c_exec, c_skip)
        alive = best > -np.inf
        alive &= ~(best < tau)
        if skip_cap >= 0:
            alive &= (prefix - budgets) <= skip_cap

        has_e, has_s = c_exec > -np.inf, c_skip > -np.inf
        with np.errstate(invalid="ignore"):
            margins[i] = np.where(has_e & has_s, np.abs(c_exec - c_skip),
                                  np.where(has_e ^ has_s, np.inf, np.nan))

        new_g = g.copy()
        new_bits = bits.copy()
        e_full = np.zeros_like(g)
        e_full[tgt] = ex
        tb = np.nonzero(take)[0]
        new_g[tb] = e_full[tb]
        new_bits[tb] = bits[tb - wi]
        new_bits[tb, i] = True
        dead = ~alive
        new_g[dead] = 0.0
        new_bits[dead] = False

        decisions[i] = np.where(alive, take.astype(np.uint8), 255)
        kept = np.where(alive, best, np.nan)
        g, bits, valid, ref = new_g, new_bits, alive, ref_new

    return DPResult(bits=bits, valid=valid, cos=kept, decisions=decisions, margins=margins,
                    states=g, ref=ref)


@dataclasses.dataclass
class BeamResult:
    bits: np.ndarray        # bool [B][k][n_items]; slot 0 is the budget's best set
    valid: np.ndarray       # bool [B][k]
    cos: np.ndarray         # float64 [B][k], NaN where invalid
    states: np.ndarray      # float32 [B][k][...] final states
    ref: np.ndarray

    def best(self) -> DPResult:
        """Slot 0 of every budget in DPResult form (no per-cell decisions or margins)."""
        B, n_items = self.bits.shape[0], self.bits.shape[2]
        return DPResult(bits=self.bits[:, 0].copy(), valid=self.valid[:, 0].copy(),
                        cos=self.cos[:, 0].copy(),
                        decisions=np.full((n_items, B), 255, dtype=np.uint8),
                        margins=np.full((n_items, B), np.nan), states=self.states[:, 0].copy(),
                        ref=self.ref)


def knapsack_dp_beam(apply_item: Callable[[int, np.ndarray], np.ndarray], n_items: int,
                     w: Sequence[int], x0: np.ndarray, n_budgets: int, beam: int,
                     tau: float = -np.inf, skip_cap: int = -1) -> BeamResult:
    """The DP with the top-``beam`` states kept per (item, budget) cell instead of one.

    Review, "Reading between the lines": an exact-knapsack or beam-search variant of the
    greedy rule shows how much headroom the one-state DP leaves.  Reading taken here: at item
    i the candidates of budget b are the skip candidates (every state kept at b) and the
    execute candidates (item i applied to every state kept at b - w_i); they are ranked by
    cosine to the reference after item i, higher first, with exact ties ordering skip
    candidates before execute candidates and then by the slot they came from; NaN ranks as
    minus infinity and such candidates are dropped; the first ``beam`` survive.  tau and the
    skip cap act as in knapsack_dp.  beam = 1 is knapsack_dp; a beam at least the number of
    subsets of any one weight keeps every subset, i.e. enumeration.
    """
    B, k = int(n_budgets), int(beam)
    assert k >= 1
    x0 = np.asarray(x0, dtype=F32)
    g = np.zeros((B, k) + x0.shape, dtype=F32)
    valid = np.zeros((B, k), dtype=bool)
    bits = np.zeros((B, k, n_items), dtype=bool)
    cosv = np.full((B, k), np.nan)
    g[0, 0] = x0
    valid[0, 0] = True
    ref = x0.copy()
    prefix = 0
    for i in range(n_items):
        wi = int(w[i])
        prefix += wi
        src = [(b, j) for b in range(max(0, B - wi)) for j in range(k) if valid[b, j]]
        rows = np.concatenate([np.stack([g[b, j] for b, j in src])
                               if src else np.zeros((0,) + x0.shape, F32), ref[None]], axis=0)
        out = apply_item(i, rows)
        ref_new = out[-1].astype(F32)
        ex = {src[m]: out[m] for m in range(len(src))}
        new_g = np.zeros_like(g)
        new_valid = np.zeros_like(valid)
        new_bits = np.zeros_like(bits)
        new_cos = np.full((B, k), np.nan)
        for b in range(B):
            cands = []  # (cos, kind 0 skip / 1 exec, slot, state, bits)
            for j in range(k):
                if valid[b, j]:
                    cands.append((g[b, j], 0, j, bits[b, j]))
            if b - wi >= 0:
                for j in range(k):
                    if (b - wi, j) in ex:
                        nb = bits[b - wi, j].copy()
                        nb[i] = True
                        cands.append((ex[(b - wi, j)], 1, j, nb))
            if not cands:
                continue
            c = cos_rows(np.stack([cd[0] for cd in cands]), ref_new)
            c = np.where(np.isnan(c), -np.inf, c)
            order = sorted(range(len(cands)), key=lambda m: (-c[m], cands[m][1], cands[m][2]))
            if skip_cap >= 0 and prefix - b > skip_cap:
                continue
            kept = 0
            for m in order:
                if kept == k or not (c[m] > -np.inf) or c[m] < tau:
                    break
                new_g[b, kept] = cands[m][0]
                new_bits[b, kept] = cands[m][3]
                new_valid[b, kept] = True
                new_cos[b, kept] = c[m]
                kept += 1
        g, valid, bits, cosv, ref = new_g, new_valid, new_bits, new_cos, ref_new
    return BeamResult(bits=bits, valid=valid, cos=cosv, states=g, ref=ref)


def pack_masks(bits: np.ndarray) -> np.ndarray:
    """bool [B][n_items] -> uint64 [B][ceil(n_items/64)], bit i of word i//64 = item i."""
    B, n = bits.shape
    words = (n + 63) // 64
    out = np.zeros((B, words), dtype=np.uint64)
    for i in range(n):
        out[:, i // 64] |= bits[:, i].astype(np.uint64) << np.uint64(i % 64)
    return out


def unpack_masks(masks: np.ndarray, n_items: int) -> np.ndarray:
    B = masks.shape[0]
    bits = np.zeros((B, n_items), dtype=bool)
    for i in range(n_items):
        bits[:, i] = ((masks[:, i // 64] >> np.uint64(i % 64)) & np.uint64(1)) == 1
    return bits


def eval_subsets(apply_item: Callable[[int, np.ndarray], np.ndarray], n_items: int,
                 x0: np.ndarray, bits: np.ndarray) -> np.ndarray:
    """cos(f^(S)(x0), f(x0)) at the last depth for each subset row of ``bits`` [R][n_items]."""
    R = bits.shape[0]
    x0 = np.asarray(x0, dtype=F32)
    rows = np.repeat(x0[None], R + 1, axis=0)
    for i in range(n_items):
        sel = np.concatenate([np.nonzero(bits[:, i])[0], [R]])
        rows[sel] = apply_item(i, rows[sel])
    return cos_rows(rows[:R], rows[R])


def brute_force(apply_item: Callable[[int, np.ndarray], np.ndarray], n_items: int,
                x0: np.ndarray):
    """Every subset of the items, by prefix sharing: returns (subset ids, final cosines).

    Subset id bit i = item i executed.  Review, "What would settle it": enumerate all layer
    subsets of a small model and compare with the DP's per-budget choice.
    """
    rows = np.asarray(x0, dtype=F32)[None].copy()
    ids = np.zeros(1, dtype=np.int64)
    for i in range(n_items):
        ex = apply_item(i, rows)
        rows = np.concatenate([rows, ex], axis=0)
        ids = np.concatenate([ids, ids | (1 << i)])
    full = (1 << n_items) - 1
    ref = rows[np.nonzero(ids == full)[0][0]]
    return ids, cos_rows(rows, ref)


# --------------------------------------------------------------------------------------
# Tokens-per-Time objective and the grid over draft length
# --------------------------------------------------------------------------------------

def tpt_value(alpha: float, gamma: int, t_draft: float, t_target: float) -> float:
    """TPT(S, gamma) = ((1 - a^(gamma+1)) / (1 - a)) / (gamma * t_draft + t_target).

    Review, "What carries the argument" (Eq. 4).  The expected-accepted-tokens factor is the
    geometric sum 1 + a + ... + a^gamma; it is summed term by term when 1 - a < 1e-6, where
    the quotient form loses precision (at a = 1 it equals gamma + 1).
    """
    a = float(alpha)
    if 1.0 - a < 1e-6:
        acc = 0.0
        p = 1.0
        for _ in range(gamma + 1):
            acc += p
            p *= a
        num = acc
    else:
        num = (1.0 - a ** (gamma + 1)) / (1.0 - a)
    return num / (gamma * float(t_draft) + float(t_target))


def tpt_select(alpha: np.ndarray, t_draft: np.ndarray, valid: np.ndarray, t_target: float,
               gamma_min: int, gamma_max: int):
    """Grid search over valid budgets and gamma in [gamma_min, gamma_max] for max TPT.

    Review, "What carries the argument" and free parameter D (grid up to a maximum draft
    length).  Ties keep the smaller budget, then the smaller gamma.  Returns (b*, gamma*,
    TPT*), or (-1, -1, NaN) when no budget is valid.
    """
    best = (-1, -1, float("nan"))
    for b in range(len(alpha)):
        if not valid[b]:
            continue
        for gm in range(gamma_min, gamma_max + 1):
            v = tpt_value(alpha[b], gm, t_draft[b], t_target)
            if best[0] < 0 or v > best[2]:
                best = (b, gm, v)
    return best


def alpha_from_cos(cos: np.ndarray) -> np.ndarray:
    """Acceptance proxy: clamp(cos, 0, 1).  The paper's history estimate (Eq. 9) is not
    printed; the cosine is the value the DP maximises (review, Lemma 4.1 discussion)."""
    a = np.clip(np.nan_to_num(np.asarray(cos, dtype=F64), nan=0.0), 0.0, 1.0)
    return a


def greedy_tokens(X: np.ndarray, w_lm: np.ndarray, eps: float):
    """Greedy next token of each token state: argmax_v (rmsnorm(x) . w_lm[v]) in float64,
    ties to the smaller v.  X [..., d], w_lm [V][d] (float32 or bf16 bits).  Returns
    (tokens [...], margin between the two largest logits [...])."""
    W = widen(w_lm).astype(F64)
    x = rmsnorm(np.asarray(X, dtype=F32), eps).astype(F64)
    logits = x.reshape(-1, x.shape[-1]) @ W.T
    tok = np.argmax(logits, axis=1)
    top2 = np.sort(logits, axis=1)[:, -2:] if W.shape[0] > 1 else np.stack(
        [np.full(len(tok), -np.inf), logits[:, 0]], axis=1)
    return tok.reshape(x.shape[:-1]), (top2[:, 1] - top2[:, 0]).reshape(x.shape[:-1])


def alpha_lm_head(states: np.ndarray, valid: np.ndarray, ref: np.ndarray, w_lm: np.ndarray,
                  eps: float) -> np.ndarray:
    """History estimate of the acceptance rate for every budget: the fraction of the r window
    tokens whose greedy token under the candidate's final state equals the full model's.

    Review, free parameters (cache window m "used for DP and acceptance estimation") and the
    circularity check (Eq. 9: a history-based estimate of alpha_S); the formula is not printed.
    Reading: compare greedy tokens through an LM head with the RMSNorm'd final states, the
    full model's tokens standing in for the accepted history.  0 where a budget is invalid.
    """
    states = np.asarray(states, dtype=F32)
    B = states.shape[0]
    if states.ndim == 2:
        states = states[:, None, :]
        ref = np.asarray(ref)[None, :]
    r = states.shape[1]
    tok, _ = greedy_tokens(states, w_lm, eps)
    tref, _ = greedy_tokens(ref, w_lm, eps)
    a = (tok == tref[None, :]).sum(axis=1).astype(F64) / r
    return np.where(np.asarray(valid, dtype=bool), a, 0.0)


@dataclasses.dataclass
class DraftVerify:
    draft: np.ndarray          # int64 [gamma] greedy tokens of the masked draft
    draft_margin: np.ndarray   # float64 [gamma] their top-2 logit gaps
    verify: np.ndarray         # int64 [gamma + 1] the target's greedy tokens on the block
    verify_margin: np.ndarray  # float64 [gamma + 1]
    accepted: int              # leading draft tokens equal to the target's


def draft_verify(shape: DecoderShape, layers, kv, x0: np.ndarray, ctx: int, bits: np.ndarray,
                 gamma: int, w_lm: np.ndarray) -> DraftVerify:
    """One self-speculative step with the chosen layer set: gamma draft tokens, then one
    verification pass of gamma + 1 tokens (review, "The reading" and "What carries the
    argument": the draft runs the selected items, the target verifies).

    Readings (the pages print no decode loop): tokens are greedy (argmax of the LM head over
    the RMSNorm'd final state, ties to the lower index); a token's input state is its LM-head
    row (tied embeddings); draft token t sits at position ctx + t and its executed Attention
    items append their key/value there, so later draft tokens attend to the cache 0..ctx-1 and
    to the earlier draft tokens' entries of the layers the draft ran; the verification runs
    every item on [x0, e(y_0), .., e(y_{gamma-1})] at positions ctx .. ctx+gamma as one causal
    block over the cache 0..ctx-1; accepted = the number of leading t with y_t equal to the
    target's token z_t.  kv is not modified.
    """
    s = shape
    hq, hkv, dh = s.n_q_heads, s.n_kv_heads, s.head_dim
    n_items = 2 * s.n_layers
    W = widen(w_lm)
    cap = ctx + gamma + 1
    caches = []
    for l in range(s.n_layers):
        kc, vc = kv[l]
        k2 = np.zeros((hkv, cap, dh), F32)
        v2 = np.zeros((hkv, cap, dh), F32)
        k2[:, :ctx] = widen(kc[:, :ctx])
        v2[:, :ctx] = widen(vc[:, :ctx])
        caches.append((k2, v2))
    wts = [{k: widen(v) for k, v in layers[l].items()} for l in range(s.n_layers)]

    def own_kv(x, w, pos):
        xn = rmsnorm(x[None], s.rms_eps)
        qkv = (xn @ w["w_qkv"].T)[0]
        k = qkv[hq * dh:(hq + hkv) * dh].reshape(hkv, dh)
        v = qkv[(hq + hkv) * dh:].reshape(hkv, dh)
        c, sn = rope_cos_sin(pos, dh, s.rope_theta)
        return rope(k, c, sn), v

    x = np.asarray(x0, F32).copy()
    inputs = [x.copy()]
    draft, dmar = [], []
    for t in range(gamma):
        pos = ctx + t
        for i in range(n_items):
            if not bits[i]:
                continue
            l, w = i // 2, wts[i // 2]
            if i % 2 == 0:
                kc, vc = caches[l]
                k, v = own_kv(x, w, pos)
                x = attention_item(x[None], w["w_qkv"], w["w_o"], kc, vc, pos, s)[0]
                kc[:, pos], vc[:, pos] = k, v
            else:
                x = mlp_item(x[None], w["w_gate_up"], w["w_down"], s)[0]
        tok, mar = greedy_tokens(x[None], W, s.rms_eps)
        draft.append(int(tok[0]))
        dmar.append(float(mar[0]))
        x = W[int(tok[0])].astype(F32).copy()
        inputs.append(x.copy())
    X = np.stack(inputs)[None]                      # [1][gamma+1][d]
    for i in range(n_items):
        l, w = i // 2, wts[i // 2]
        if i % 2 == 0:
            X = attention_item_window(X, w["w_qkv"], w["w_o"], kv[l][0], kv[l][1], ctx, s)
        else:
            M, r, d = X.shape
            X = mlp_item(X.reshape(M * r, d), w["w_gate_up"], w["w_down"], s).reshape(M, r, d)
    ver, vmar = greedy_tokens(X[0], W, s.rms_eps)
    acc = 0
    while acc < gamma and draft[acc] == int(ver[acc]):
        acc += 1
    return DraftVerify(draft=np.array(draft, dtype=np.int64), draft_margin=np.array(dmar),
                       verify=np.asarray(ver, dtype=np.int64), verify_margin=np.asarray(vmar),
                       accepted=acc)


# --------------------------------------------------------------------------------------
# One full solve
# --------------------------------------------------------------------------------------

@dataclasses.dataclass
class SolveResult:
    dp: DPResult
    t: np.ndarray           # float64 [n_items] latencies
    w: np.ndarray           # int64 [n_items] weights
    masks: np.ndarray       # uint64 [B][words]
    t_draft: np.ndarray     # float64 [B]
    t_target: float
    best_budget: int
    best_gamma: int
    best_tpt: float
    alpha: np.ndarray = None  # float64 [B] acceptance estimate the TPT grid used


def solve(shape: DecoderShape, layers, kv, x0: np.ndarray, ctx: int, latency: dict,
          n_budgets: int, gamma: Sequence[int], tau: float = -np.inf, skip_cap: int = -1,
          per_item: Optional[Sequence[float]] = None, cache_widened: bool = False,
          apply_item: Optional[Callable] = None,
          w_lm: Optional[np.ndarray] = None, beam: int = 1) -> SolveResult:
    """Latencies -> weights -> DP -> per-budget draft latency -> TPT grid, for one sequence.

    t_Draft(S) = fixed + sum_{i in S} t_i and t_Target = fixed + sum_i t_i: one draft pass
    runs the kept items, one verification pass runs all of them (readings; the page defines
    TPT in terms of both but prints no formula for them).  x0 is [d] (one token) or [r][d]
    (an r-token window).  With ``w_lm`` the TPT grid uses alpha_lm_head, else clamp(cos).
    ``beam`` > 1 runs knapsack_dp_beam and uses each budget's best set.
    """
    n_items = 2 * shape.n_layers
    t = item_latencies(shape.n_layers, ctx, latency["attn_base"], latency["attn_per_token"],
                       latency["mlp"], per_item)
    w = item_weights(t, n_budgets)
    fn = apply_item if apply_item is not None else DecoderItems(shape, layers, kv, ctx,
                                                                 cache_widened)
    if beam > 1:
        dp = knapsack_dp_beam(fn, n_items, w, x0, n_budgets, beam, tau, skip_cap).best()
    else:
        dp = knapsack_dp(fn, n_items, w, x0, n_budgets, tau, skip_cap)
    fixed = float(latency.get("fixed", 0.0))
    t_draft = np.array([fixed + float(np.sum(t[dp.bits[b]])) for b in range(n_budgets)])
    t_target = fixed + float(np.sum(t))
    if w_lm is not None:
        alpha = alpha_lm_head(dp.states, dp.valid, dp.ref, w_lm, shape.rms_eps)
    else:
        alpha = alpha_from_cos(dp.cos)
    bb, bg, bt = tpt_select(alpha, t_draft, dp.valid, t_target, int(gamma[0]), int(gamma[1]))
    return SolveResult(dp=dp, t=t, w=w, masks=pack_masks(dp.bits), t_draft=t_draft,
                       t_target=t_target, best_budget=bb, best_gamma=bg, best_tpt=bt,
                       alpha=alpha)

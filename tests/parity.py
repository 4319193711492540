"""Tie-aware comparison of a GPU solve with the oracle's (rules P1-P4).

Several results are correct wherever execute and skip are within the tolerance band beta of
each other: either choice is a valid outcome of the DP, and everything computed downstream
of it may legitimately differ.  So:
  P1  clean cells (oracle margin >= beta and both predecessor cells clean) must carry the
      same decision on the GPU;
  P2  every valid GPU budget's cosine must equal the oracle's forward of the GPU's own mask
      within beta (holds everywhere, excused or not);
  P3  valid sets must agree except at excused budgets;
  P4  the chosen (b, gamma) must agree unless the GPU's pick is within the band of the
      oracle's best TPT.
Item weights and per-budget draft latencies of identical masks are compared exactly.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from oracle import knapspec_oracle as ko


@dataclasses.dataclass
class ParityReport:
    cells: int
    clean: int
    excused: int
    mismatched_clean: int
    p2_max_err: float
    p3_bad: int
    p4_ok: bool
    same_pick: bool
    max_cos_diff_same_mask: float

    def line(self) -> str:
        return (f"cells={self.cells} clean={self.clean} excused={self.excused} "
                f"({self.excused / max(1, self.cells):.1%}) clean_mismatch={self.mismatched_clean} "
                f"P2max={self.p2_max_err:.2e} P3bad={self.p3_bad} P4={'ok' if self.p4_ok else 'FAIL'} "
                f"same_pick={self.same_pick} max|dcos|same-mask={self.max_cos_diff_same_mask:.2e}")


def clean_cells(oracle: ko.SolveResult, beta: float) -> np.ndarray:
    """bool [n_items][B]: cell decisions that no near-tie upstream can legitimately change."""
    dp = oracle.dp
    n_items, B = dp.decisions.shape
    clean = np.zeros((n_items, B), dtype=bool)
    prev = np.ones(B, dtype=bool)  # the initial state is exact
    for i in range(n_items):
        w = int(oracle.w[i])
        m = dp.margins[i]
        ok = ~(m < beta)  # NaN (no candidate) and inf (one candidate) count as clean
        pred_skip = prev
        pred_exec = np.ones(B, dtype=bool)
        pred_exec[w:] = prev[: B - w] if w < B else pred_exec[w:]
        clean[i] = ok & pred_skip & pred_exec
        prev = clean[i]
    return clean


def compare(oracle: ko.SolveResult, gpu_res, seq: int, beta: float, apply_item, x0,
            gamma, n_items: int, p2_cos=None) -> ParityReport:
    """``p2_cos`` (optional, float64 [B]): the oracle's cosine of every valid GPU budget's
    mask, already computed (e.g. by LockstepSubsets alongside the DP); otherwise P2 runs
    eval_subsets here."""
    dp = oracle.dp
    B = dp.valid.shape[0]
    assert np.array_equal(gpu_res.item_weight[seq], oracle.w.astype(np.int32)), \
        (gpu_res.item_weight[seq], oracle.w)
    clean = clean_cells(oracle, beta)
    dec_g = gpu_res.decisions[seq] if gpu_res.decisions is not None else None
    mism = 0
    if dec_g is not None:
        mism = int(np.sum((dec_g != dp.decisions) & clean))
    valid_g = gpu_res.valid[seq].astype(bool)
    final_clean = clean[-1]
    p3_bad = int(np.sum((valid_g != dp.valid) & final_clean))

    # P2: the oracle's forward of every valid GPU mask
    gbits = ko.unpack_masks(gpu_res.masks[seq], n_items)
    vb = np.nonzero(valid_g)[0]
    p2 = 0.0
    ev = np.full(B, np.nan)
    if len(vb):
        ev[vb] = (np.asarray(p2_cos)[vb] if p2_cos is not None
                  else ko.eval_subsets(apply_item, n_items, x0, gbits[vb]))
        p2 = float(np.max(np.abs(ev[vb] - gpu_res.cos[seq][vb].astype(np.float64))))
    same_mask = valid_g & dp.valid & np.all(gbits == dp.bits, axis=1)
    dcos = 0.0
    if same_mask.any():
        dcos = float(np.max(np.abs(gpu_res.cos[seq][same_mask] - dp.cos[same_mask])))
        # identical masks must have identical draft latencies
        assert np.allclose(gpu_res.t_draft[seq][same_mask], oracle.t_draft[same_mask],
                           rtol=0, atol=1e-9 * max(1.0, oracle.t_target))

    # P4
    bg, gg = int(gpu_res.best_budget[seq]), int(gpu_res.best_gamma[seq])
    same_pick = (bg, gg) == (oracle.best_budget, oracle.best_gamma)
    p4 = same_pick
    if not same_pick and bg >= 0 and oracle.best_budget >= 0:
        a_g = min(1.0, max(0.0, ev[bg] + beta))
        lhs = ko.tpt_value(a_g, gg, gpu_res.t_draft[seq][bg], oracle.t_target)
        a_o = min(1.0, max(0.0, dp.cos[oracle.best_budget] - beta))
        rhs = ko.tpt_value(a_o, oracle.best_gamma, oracle.t_draft[oracle.best_budget],
                           oracle.t_target)
        p4 = lhs >= rhs
    cells = int(np.sum(dp.decisions != 255) + np.sum(dp.decisions == 255))
    return ParityReport(cells=cells, clean=int(clean.sum()), excused=int((~clean).sum()),
                        mismatched_clean=mism, p2_max_err=p2, p3_bad=p3_bad, p4_ok=bool(p4),
                        same_pick=bool(same_pick), max_cos_diff_same_mask=dcos)


def forward_states(apply_item, n_items: int, x0, bits: np.ndarray):
    """The oracle's final states for each subset row of ``bits`` [R][n_items] and the full
    model's (every item), from the same input x0 ([d] or [r][d])."""
    R = bits.shape[0]
    x0 = np.asarray(x0, dtype=np.float32)
    rows = np.repeat(x0[None], R + 1, axis=0)
    for i in range(n_items):
        sel = np.concatenate([np.nonzero(bits[:, i])[0], [R]])
        rows[sel] = apply_item(i, rows[sel])
    return rows[:R], rows[R]


@dataclasses.dataclass
class AlphaReport:
    budgets: int
    tokens: int
    excused_tokens: int
    mismatched_tokens: int
    alpha_mismatch: int

    def line(self) -> str:
        return (f"budgets={self.budgets} tokens={self.tokens} excused={self.excused_tokens} "
                f"token_mismatch={self.mismatched_tokens} alpha_mismatch={self.alpha_mismatch}")


def compare_alpha(gpu_res, seq: int, apply_item, x0, w_lm, eps: float, band: float,
                  n_items: int) -> AlphaReport:
    """P5: every valid GPU budget's greedy tokens (and the full model's) against the oracle's
    greedy tokens of the oracle's forward of the GPU's own mask; a window token whose oracle
    top-2 logit margin (for the budget or for the full model) is below ``band`` is excused.
    The GPU's alpha must equal the match fraction of its own tokens, and equal the oracle's
    wherever no token of the budget is excused."""
    valid = gpu_res.valid[seq].astype(bool)
    vb = np.nonzero(valid)[0]
    tok_g = gpu_res.tokens(seq)                   # [B+1][r]
    r = tok_g.shape[1]
    B = valid.shape[0]
    bits = ko.unpack_masks(gpu_res.masks[seq], n_items)[vb]
    st, ref = forward_states(apply_item, n_items, x0, bits)
    st = st.reshape(len(vb), r, -1)
    ref = np.asarray(ref).reshape(r, -1)
    tok_o, mar_o = ko.greedy_tokens(st, w_lm, eps)
    tref_o, mref_o = ko.greedy_tokens(ref, w_lm, eps)
    clean_ref = mref_o >= band
    # the full model's tokens
    mism = int(np.sum((tok_g[B] != tref_o) & clean_ref))
    excused = int(np.sum(~clean_ref))
    alpha_bad = 0
    for k, b in enumerate(vb):
        clean = (mar_o[k] >= band) & clean_ref
        excused += int(np.sum(~clean))
        mism += int(np.sum((tok_g[b] != tok_o[k]) & clean))
        # alphas are match counts over r, returned in float32
        a_self = float(np.sum(tok_g[b] == tok_g[B])) / r
        if abs(float(gpu_res.alpha[seq][b]) - a_self) > 1e-6:
            alpha_bad += 1
        if clean.all():
            a_orc = float(np.sum(tok_o[k] == tref_o)) / r
            alpha_bad += int(abs(float(gpu_res.alpha[seq][b]) - a_orc) > 1e-6)
    assert np.all(gpu_res.alpha[seq][~valid] == 0.0)
    assert np.all(tok_g[np.nonzero(~valid)[0]] == -1)
    return AlphaReport(budgets=len(vb), tokens=(len(vb) + 1) * r, excused_tokens=excused,
                       mismatched_tokens=mism, alpha_mismatch=alpha_bad)

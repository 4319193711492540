"""Pins for the oracle's knapsack DP skeleton: indices, masks, ties, pruning.

With additive items F_i(x) = x + u_i, where x0 and all u_i are mutually orthogonal, the
cosine of a subset state x_S = x0 + sum_{k in S} u_k with the full-model state X^(i) is
sqrt(|x0|^2 + V_S) / |X^(i)|, V_S = sum_{k in S} |u_k|^2 -- monotone in V_S.  The greedy
cosine DP is then exactly the textbook exact-weight 0/1 knapsack
    V[i, b] = max(V[i-1, b], V[i-1, b - w_i] + |u_i|^2),
which the tests below implement independently (plain Python, no oracle code).
"""
import numpy as np
import pytest

from oracle import knapspec_oracle as ko


def _orthogonal_items(n_items, d, seed):
    rng = np.random.default_rng(seed)
    Q, _ = np.linalg.qr(rng.standard_normal((d, n_items + 1)))
    x0 = (Q[:, 0] * rng.uniform(0.5, 1.5)).astype(np.float32)
    norms = rng.uniform(0.2, 2.0, size=n_items)
    U = (Q[:, 1:] * norms).T.astype(np.float32)  # [n_items][d]
    return x0, U


def _additive(U):
    return lambda i, X: (X + U[i][None, :]).astype(np.float32)


def textbook_knapsack(values, weights, B, keep=None):
    """Exact-weight 0/1 knapsack over budgets 0..B-1 with set recovery by carrying sets.

    keep(i, b, V) -> bool optionally drops cells after item i (pruning rules)."""
    NEG = float("-inf")
    V = [0.0] + [NEG] * (B - 1)
    S = [frozenset()] + [None] * (B - 1)
    for i, (v, w) in enumerate(zip(values, weights)):
        nV, nS = list(V), list(S)
        for b in range(B):
            if b - w >= 0 and V[b - w] != NEG:
                cand = V[b - w] + v
                if cand > V[b]:
                    nV[b], nS[b] = cand, S[b - w] | {i}
        if keep is not None:
            for b in range(B):
                if nV[b] != NEG and not keep(i, b, nV[b]):
                    nV[b], nS[b] = NEG, None
        V, S = nV, nS
    return V, S


def _v_of(bits_row, U):
    return float(sum(float(np.dot(U[i].astype(np.float64), U[i])) for i in np.nonzero(bits_row)[0]))


@pytest.mark.parametrize("seed,n_items,B", [(0, 10, 12), (1, 14, 40), (2, 16, 64), (3, 9, 6)])
def test_additive_dp_is_textbook_knapsack(seed, n_items, B):
    d = 48
    x0, U = _orthogonal_items(n_items, d, seed)
    rng = np.random.default_rng(100 + seed)
    w = rng.integers(1, 5, size=n_items)
    res = ko.knapsack_dp(_additive(U), n_items, w, x0, B)
    vals = [float(np.dot(U[i].astype(np.float64), U[i])) for i in range(n_items)]
    V, S = textbook_knapsack(vals, list(w), B)
    a = float(np.dot(x0.astype(np.float64), x0))
    ref_norm2 = a + sum(vals)
    for b in range(B):
        assert res.valid[b] == (V[b] != float("-inf")), b
        if not res.valid[b]:
            continue
        got = set(np.nonzero(res.bits[b])[0].tolist())
        assert got == set(S[b]), (b, got, S[b])
        assert sum(int(w[i]) for i in got) == b
        assert res.cos[b] == pytest.approx(np.sqrt((a + V[b]) / ref_norm2), abs=2e-6)


def test_paper_skipped_weight_index_gives_same_sets():
    """Referee minor comment 2: the paper indexes cells by skipped weight j (skip moves
    j -> j + w, execute keeps j).  With sum(w) <= B-1 no budget is truncated and the two
    conventions must produce the same candidate set for b = P - j."""
    n_items, d = 12, 40
    x0, U = _orthogonal_items(n_items, d, 7)
    w = np.random.default_rng(8).integers(1, 4, size=n_items)
    K = int(w.sum())
    F = _additive(U)
    # paper convention, written here from its description only
    g = {0: x0.astype(np.float32)}
    sets = {0: frozenset()}
    ref = x0.astype(np.float32)
    for i in range(n_items):
        ref_new = F(i, ref[None])[0]
        ng, ns = {}, {}
        for j in range(K + 1):
            cands = []
            if j in g:  # execute item i: skipped weight unchanged
                e = F(i, g[j][None])[0]
                cands.append((ko.cos_rows(e[None], ref_new)[0], 1, e, sets[j] | {i}))
            if j - w[i] in g:  # skip item i: skipped weight grows by w_i
                s = g[j - w[i]]
                cands.append((ko.cos_rows(s[None], ref_new)[0], 0, s, sets[j - w[i]]))
            if not cands:
                continue
            # skip wins exact ties (the same reading as the oracle)
            cands.sort(key=lambda c: (c[0], -c[1]))
            best = cands[-1]
            if len(cands) == 2 and cands[0][0] == cands[1][0]:
                best = [c for c in cands if c[1] == 0][0]
            ng[j], ns[j] = best[2], best[3]
        g, sets, ref = ng, ns, ref_new
    res = ko.knapsack_dp(F, n_items, w, x0, K + 1)
    for j, st in sets.items():
        b = K - j
        assert res.valid[b]
        assert set(np.nonzero(res.bits[b])[0].tolist()) == set(st)
    assert int(res.valid.sum()) == len(sets)


def test_tau_pruning_matches_textbook_threshold():
    n_items, d, B = 12, 40, 30
    x0, U = _orthogonal_items(n_items, d, 11)
    w = np.random.default_rng(12).integers(1, 4, size=n_items)
    vals = [float(np.dot(U[i].astype(np.float64), U[i])) for i in range(n_items)]
    a = float(np.dot(x0.astype(np.float64), x0))
    prefix_v = np.cumsum(vals)
    tau = 0.8

    def keep(i, b, v):  # cos after item i = sqrt((a + v) / (a + sum_{k<=i} |u_k|^2))
        return np.sqrt((a + v) / (a + prefix_v[i])) >= tau

    V, S = textbook_knapsack(vals, list(w), B, keep)
    res = ko.knapsack_dp(_additive(U), n_items, w, x0, B, tau=tau)
    for b in range(B):
        assert res.valid[b] == (V[b] != float("-inf")), b
        if res.valid[b]:
            assert set(np.nonzero(res.bits[b])[0].tolist()) == set(S[b])
            assert res.cos[b] >= tau


def test_skip_cap_matches_textbook_constraint():
    n_items, d, B = 12, 40, 40
    x0, U = _orthogonal_items(n_items, d, 21)
    w = np.random.default_rng(22).integers(1, 4, size=n_items)
    vals = [float(np.dot(U[i].astype(np.float64), U[i])) for i in range(n_items)]
    prefix_w = np.cumsum(w)
    cap = int(prefix_w[-1]) // 2

    def keep(i, b, v):  # skipped weight so far = prefix - used
        return prefix_w[i] - b <= cap

    V, S = textbook_knapsack(vals, list(w), B, keep)
    res = ko.knapsack_dp(_additive(U), n_items, w, x0, B, skip_cap=cap)
    for b in range(B):
        assert res.valid[b] == (V[b] != float("-inf")), b
        if res.valid[b]:
            assert set(np.nonzero(res.bits[b])[0].tolist()) == set(S[b])


def test_tau_above_one_prunes_everything():
    x0, U = _orthogonal_items(6, 16, 3)
    res = ko.knapsack_dp(_additive(U), 6, [1] * 6, x0, 8, tau=1.5)
    assert not res.valid.any()
    assert np.all(res.decisions[-1] == 255)


def test_decisions_backtrack_to_carried_masks():
    """Recover each set from the per-cell decisions by walking back (the paper's backtracking
    idea, Algorithm 2 in referee minor comment 4) and compare with the carried masks."""
    n_items, d, B = 14, 40, 25
    x0, U = _orthogonal_items(n_items, d, 31)
    w = np.random.default_rng(32).integers(1, 4, size=n_items)
    res = ko.knapsack_dp(_additive(U), n_items, w, x0, B)
    for b0 in range(B):
        if not res.valid[b0]:
            continue
        b, items = b0, set()
        for i in range(n_items - 1, -1, -1):
            dcs = res.decisions[i][b]
            assert dcs in (0, 1)
            if dcs == 1:
                items.add(i)
                b -= int(w[i])
        assert b == 0
        assert items == set(np.nonzero(res.bits[b0])[0].tolist())


def test_nan_input_makes_cells_invalid():
    x0, U = _orthogonal_items(6, 16, 5)
    x0 = x0.copy()
    x0[3] = np.nan
    res = ko.knapsack_dp(_additive(U), 6, [1] * 6, x0, 8)
    assert not res.valid.any()


def test_mask_pack_roundtrip():
    rng = np.random.default_rng(0)
    bits = rng.random((7, 160)) < 0.5
    masks = ko.pack_masks(bits)
    assert masks.shape == (7, 3)
    assert np.array_equal(ko.unpack_masks(masks, 160), bits)
    assert int(masks[0, 0]) & 1 == int(bits[0, 0])
    assert (int(masks[0, 2]) >> 31) & 1 == int(bits[0, 159])

"""Pins of the sparse-index oracle (CPU only), and planted mistakes that the pins must catch.

The estimator is a reading of the pages (they name none), so it is pinned by closed forms
of its own definition that any plausible slip breaks: equal keys (ties and the diagonal),
block scores built to grow with the key block (ranking direction, causality), probe
importances of equal keys (causal softmax normalisation), planted blocks and columns, list
counts and order, and the GQA head map.
"""

import numpy as np
import pytest

from oracle import sparse_index as X

RNG = np.random.default_rng(12345)
BLK = 64


def _qk(B, L, Hq, Hkv, D, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal((B, L, Hq, D)), r.standard_normal((B, L, Hkv, D))


def _lists(blk_ptr, blk_idx, B, Hq, nqb):
    return [[blk_idx[blk_ptr[(b * Hq + h) * nqb + qb]:blk_ptr[(b * Hq + h) * nqb + qb + 1]]
             for qb in range(nqb)] for b in range(B) for h in range(Hq)]


def test_pooled_rows_closed_forms():
    x = np.arange(1, 131, dtype=np.float64)[:, None] * np.ones((1, 3))   # rows 1..130
    p = X.pooled_rows(x, 64)
    assert np.allclose(p[:, 0], [32.5, 96.5, 129.5])                     # last group: rows 129, 130


def test_equal_keys_pick_diagonal_and_lowest_blocks():
    """All keys equal: every causal block scores the same, so the ties go to the lowest ids and
    the diagonal block is always in."""
    B, L, Hq, D, topk = 1, 6 * BLK, 2, 8, 3
    q = RNG.standard_normal((B, L, Hq, D))
    k = np.tile(RNG.standard_normal((1, 1, 1, D)), (B, L, Hq, 1))
    bp, bi, _, _, _, _ = X.build_index(q, k, 0.3, topk, 4)
    for lists in _lists(bp, bi, B, Hq, 6):
        for qb, ids in enumerate(lists):
            expect = sorted(set(list(range(min(topk - 1, qb))) + [qb]))
            assert list(ids) == expect


def test_block_scores_grow_with_key_block():
    """Query rows e0, key rows of block kb equal (kb + 1) * e0: the block score is
    scale * (kb + 1), so the top blocks are the latest causal ones."""
    B, L, Hq, D, topk, scale = 1, 8 * BLK, 1, 4, 3, 0.5
    q = np.zeros((B, L, Hq, D)); q[..., 0] = 1.0
    k = np.zeros((B, L, Hq, D))
    for kb in range(8):
        k[0, kb * BLK:(kb + 1) * BLK, 0, 0] = kb + 1
    sc = X.block_scores(q[0, :, 0], k[0, :, 0], scale, BLK)
    for qb in range(8):
        assert np.allclose(sc[qb, :qb + 1], scale * np.arange(1, qb + 2))
        assert np.all(np.isneginf(sc[qb, qb + 1:]))
    bp, bi, _, _, _, _ = X.build_index(q, k, scale, topk, 4)
    for qb, ids in enumerate(_lists(bp, bi, B, Hq, 8)[0]):
        assert list(ids) == list(range(max(0, qb - topk + 1), qb + 1))


def test_planted_block_is_selected():
    B, L, Hq, D = 1, 10 * BLK, 1, 16
    q, k = _qk(B, L, Hq, 1, D, 7)
    qb, kb_star = 9, 3
    qmean = q[0, qb * BLK:(qb + 1) * BLK, 0].mean(axis=0)
    k[0, kb_star * BLK:(kb_star + 1) * BLK, 0] = 20.0 * qmean / np.linalg.norm(qmean)
    bp, bi, _, _, _, _ = X.build_index(q, k, 0.25, 2, 4)
    assert list(_lists(bp, bi, B, Hq, 10)[0][qb]) == [kb_star, qb]


def test_probe_importance_equal_keys_closed_form():
    """Equal keys: probe row r is uniform over keys j <= r, so importance_j is the sum of
    1/(r+1) over probe rows r >= j."""
    L, D, P = 150, 8, 64
    q = RNG.standard_normal((L, D))
    k = np.tile(RNG.standard_normal((1, D)), (L, 1))
    imp = X.probe_importance(q, k, 0.7, P)
    rows = np.arange(L - P, L)
    expect = np.array([np.sum(1.0 / (rows[rows >= j] + 1)) for j in range(L)])
    assert np.allclose(imp, expect, rtol=1e-12, atol=1e-14)
    assert np.isclose(imp.sum(), P)


def test_probe_uses_all_rows_when_short():
    L, D = 40, 4
    q = RNG.standard_normal((L, D))
    k = np.tile(RNG.standard_normal((1, D)), (L, 1))
    imp = X.probe_importance(q, k, 1.0, 64)
    assert np.isclose(imp.sum(), L)
    assert np.isclose(imp[0], np.sum(1.0 / np.arange(1, L + 1)))


def test_equal_keys_columns_go_to_lowest_indices():
    """Equal keys: importance is flat over the keys every probe row sees and falls after, so
    the ties go to the lowest indices."""
    B, L, Hq, D = 1, 300, 1, 8
    q = RNG.standard_normal((B, L, Hq, D))
    k = np.tile(RNG.standard_normal((1, 1, 1, D)), (B, L, Hq, 1))
    _, _, cp, ci, _, _ = X.build_index(q, k, 0.5, 4, 10)
    assert list(ci[cp[0]:cp[1]]) == list(range(10))


def test_planted_column_is_selected():
    B, L, Hq, D = 1, 500, 1, 16
    q, k = _qk(B, L, Hq, 1, D, 11)
    jstar = 77
    qm = q[0, L - 64:, 0].mean(axis=0)
    k[0, jstar, 0] = 60.0 * qm / np.dot(qm, qm)         # scale * <q_mean, k_j*> = 15
    _, _, cp, ci, _, imp = X.build_index(q, k, 0.25, 4, 1)
    assert list(ci[cp[0]:cp[1]]) == [jstar]
    assert imp[0, 0, jstar] > 0.5 * 64 and imp[0, 0, jstar] == imp[0, 0].max()


def test_counts_order_and_causality():
    B, L, Hq, Hkv, D, topk, ncol = 2, 5 * BLK + 17, 4, 2, 16, 4, 50
    q, k = _qk(B, L, Hq, Hkv, D, 3)
    bp, bi, cp, ci, _, _ = X.build_index(q, k, 0.2, topk, ncol)
    nqb = 6
    assert bp.size == B * Hq * nqb + 1 and cp.size == B * Hq + 1
    for lists in _lists(bp, bi, B, Hq, nqb):
        for qb, ids in enumerate(lists):
            assert ids.size == X.block_count(qb, topk)
            assert np.all(np.diff(ids) > 0) and ids[-1] == qb and ids[0] >= 0
    for bh in range(B * Hq):
        cols = ci[cp[bh]:cp[bh + 1]]
        assert cols.size == ncol and np.all(np.diff(cols) > 0) and cols[-1] < L


def test_gqa_head_map_contiguous_groups():
    """KV head 0 carries a planted block, KV head 1 does not: only query heads 0..g-1 (the
    contiguous group of KV head 0) select it."""
    B, L, Hq, Hkv, D = 1, 6 * BLK, 4, 2, 16
    q, k = _qk(B, L, Hq, Hkv, D, 5)
    k *= 0.01
    q[0, 5 * BLK:, :, :] = 1.0
    k[0, 2 * BLK:3 * BLK, 0, :] = 1.0
    bp, bi, _, _, _, _ = X.build_index(q, k, 0.25, 2, 4)
    lists = _lists(bp, bi, B, Hq, 6)
    assert [list(lists[h][5]) for h in range(Hq)][:2] == [[2, 5], [2, 5]]
    assert all(2 not in list(lists[h][5]) for h in (2, 3))


def test_slash_importance_sums_to_probe_rows():
    """Each probe row's probabilities sum to 1 and every visible (row, key) pair lies on
    exactly one line (offset row - key >= 0), so the importances sum to the probe size."""
    L, D = 300, 8
    q, k = RNG.standard_normal((L, D)), RNG.standard_normal((L, D))
    imp = X.slash_importance(q, k, 0.4, 64)
    assert np.isclose(imp.sum(), 64.0, rtol=1e-12)
    assert np.all(imp >= 0)


def test_slash_importance_single_probe_row_reverses_columns():
    """With one probe row r = L - 1, line o meets key L - 1 - o only: the slash importances
    are the column importances reversed."""
    L, D = 120, 6
    q, k = RNG.standard_normal((L, D)), RNG.standard_normal((L, D))
    s = X.slash_importance(q, k, 0.8, 1)
    c = X.probe_importance(q, k, 0.8, 1)
    assert np.allclose(s, c[::-1], rtol=1e-13, atol=1e-15)


def test_slash_importance_equal_keys_closed_form():
    """Equal keys: probe row r is uniform over keys 0..r, so line o collects 1/(r+1) from every
    probe row r >= o."""
    L, D, P = 150, 8, 64
    q = RNG.standard_normal((L, D))
    k = np.tile(RNG.standard_normal((1, D)), (L, 1))
    imp = X.slash_importance(q, k, 0.7, P)
    rows = np.arange(L - P, L)
    expect = np.array([np.sum(1.0 / (rows[rows >= o] + 1)) for o in range(L)])
    assert np.allclose(imp, expect, rtol=1e-12, atol=1e-14)


def test_planted_slash_is_selected():
    """Key r - o* made parallel to query row r for every probe row r: line o* carries most of
    each probe row's mass and is the top offset."""
    B, L, Hq, D, ostar = 1, 400, 1, 32, 37
    q, k = _qk(B, L, Hq, 1, D, 21)
    k *= 0.1
    for r in range(L - 64, L):
        k[0, r - ostar, 0] = 40.0 * q[0, r, 0] / np.dot(q[0, r, 0], q[0, r, 0])
    cp, ci, sp, si, cimp, simp = X.build_vslash_index(q, k, 0.25, 4, 3)
    assert ostar in list(si[sp[0]:sp[1]])
    assert simp[0, 0].argmax() == ostar and simp[0, 0, ostar] > 0.5 * 64
    assert list(ci[cp[0]:cp[1]]) == list(X.select_columns(cimp[0, 0], 4))


def test_vslash_counts_and_order():
    B, L, Hq, Hkv, D = 2, 200, 4, 2, 8
    q, k = _qk(B, L, Hq, Hkv, D, 22)
    cp, ci, sp, si, _, _ = X.build_vslash_index(q, k, 0.3, 17, 9)
    for bh in range(B * Hq):
        offs = si[sp[bh]:sp[bh + 1]]
        assert offs.size == 9 and np.all(np.diff(offs) > 0) and offs[0] >= 0 and offs[-1] < L
        assert ci[cp[bh]:cp[bh + 1]].size == 17


# ---- planted mistakes: each must make some pin above fail ------------------------------------

def _pins():
    return [test_pooled_rows_closed_forms, test_equal_keys_pick_diagonal_and_lowest_blocks,
            test_block_scores_grow_with_key_block, test_planted_block_is_selected,
            test_probe_importance_equal_keys_closed_form, test_probe_uses_all_rows_when_short,
            test_equal_keys_columns_go_to_lowest_indices, test_planted_column_is_selected,
            test_counts_order_and_causality, test_gqa_head_map_contiguous_groups,
            test_slash_importance_sums_to_probe_rows,
            test_slash_importance_single_probe_row_reverses_columns,
            test_slash_importance_equal_keys_closed_form, test_planted_slash_is_selected,
            test_vslash_counts_and_order]


def _some_pin_fails():
    for pin in _pins():
        try:
            pin()
        except Exception:
            return True
    return False


def _sel_blocks_ascending(scores_row, qb, topk):
    others = sorted(range(qb), key=lambda kb: (scores_row[kb], kb))
    return np.asarray(sorted(others[:max(0, topk - 1)] + [qb]), np.int32)


def _sel_blocks_ties_high(scores_row, qb, topk):
    others = sorted(range(qb), key=lambda kb: (-scores_row[kb], -kb))
    return np.asarray(sorted(others[:max(0, topk - 1)] + [qb]), np.int32)


def _sel_blocks_no_diagonal(scores_row, qb, topk):
    others = sorted(range(qb + 1), key=lambda kb: (-scores_row[kb], kb))
    return np.asarray(sorted(others[:topk]), np.int32)


def _probe_noncausal(q_head, k_head, scale, probe):
    L = q_head.shape[0]
    rows = np.arange(max(0, L - probe), L)
    s = scale * (q_head[rows] @ k_head.T)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return p.sum(axis=0)


def _probe_first_rows(q_head, k_head, scale, probe):
    L = q_head.shape[0]
    rows = np.arange(0, min(probe, L))
    s = scale * (q_head[rows] @ k_head.T)
    s[np.arange(L)[None, :] > rows[:, None]] = -np.inf
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return p.sum(axis=0)


def _probe_unnormalised(q_head, k_head, scale, probe):
    L = q_head.shape[0]
    rows = np.arange(max(0, L - probe), L)
    s = scale * (q_head[rows] @ k_head.T)
    s[np.arange(L)[None, :] > rows[:, None]] = -np.inf
    return np.exp(s - s.max(axis=1, keepdims=True)).sum(axis=0)


def _cols_ties_high(importance, n_cols):
    order = sorted(range(importance.shape[0]), key=lambda j: (-importance[j], -j))
    return np.asarray(sorted(order[:n_cols]), np.int32)


def _pool_first_row(x, block):
    n = -(-x.shape[0] // block)
    return np.stack([x[i * block] for i in range(n)]).astype(np.float64)


def _slash_mutant(key_of, rows_of=None):
    def imp_fn(q_head, k_head, scale, probe):
        L = q_head.shape[0]
        rows = np.arange(max(0, L - probe), L) if rows_of is None else rows_of(L, probe)
        s = scale * (q_head[rows] @ k_head.T)
        s[np.arange(L)[None, :] > rows[:, None]] = -np.inf
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        imp = np.zeros(L)
        for a, r in enumerate(rows):
            for o in range(L):
                j = key_of(r, o)
                if 0 <= j < L:
                    imp[o] += p[a, j]
        return imp
    return imp_fn


MUTANTS = {
    "blocks_ascending": ("select_blocks", _sel_blocks_ascending),
    "blocks_ties_high": ("select_blocks", _sel_blocks_ties_high),
    "blocks_no_forced_diagonal": ("select_blocks", _sel_blocks_no_diagonal),
    "probe_noncausal": ("probe_importance", _probe_noncausal),
    "probe_first_rows": ("probe_importance", _probe_first_rows),
    "probe_unnormalised": ("probe_importance", _probe_unnormalised),
    "columns_ties_high": ("select_columns", _cols_ties_high),
    "pool_first_row": ("pooled_rows", _pool_first_row),
    "slash_above_diagonal": ("slash_importance", _slash_mutant(lambda r, o: r + o)),
    "slash_off_by_one": ("slash_importance", _slash_mutant(lambda r, o: r - o - 1)),
    "slash_first_rows": ("slash_importance",
                         _slash_mutant(lambda r, o: r - o, lambda L, P: np.arange(min(P, L)))),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    fn, bad = MUTANTS[name]
    monkeypatch.setattr(X, fn, bad)
    assert _some_pin_fails(), f"no pin catches the mutant {name}"

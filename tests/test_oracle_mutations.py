"""Planted mistakes in the oracle (CPU only): each one must make at least one pin fail.

Every mutant replaces ONE named step of oracle/attention.py with a plausible error (a dropped
term, a wrong sign or index, a transposed operand, a wrong mask boundary, an intersection in
place of a union, a missing normalisation). The pins are run against the mutated oracle; the
test passes only if some pin then fails, which shows the pins can see that class of mistake.
"""

import numpy as np
import pytest

from oracle import attention as A
import tests.test_oracle_pins as P


def _pins():
    """Every pin in test_oracle_pins as a zero-argument callable."""
    g = P._golden()
    calls = []
    calls += [lambda c=c: P.test_golden_dense(c) for c in g["cases"]]
    calls += [lambda c=c: P.test_golden_blocksparse(c) for c in g["blocksparse_cases"]]
    calls += [lambda c=c: P.test_golden_combine(c) for c in g["combine_cases"]]
    calls += [lambda c=c: P.test_bruteforce_dense(c) for c in P.BF_CASES]
    calls += [lambda s=s: P.test_bruteforce_blocksparse(s) for s in range(3)]
    calls += [P.test_uniform_keys_give_prefix_means, P.test_constant_values_give_constant_output,
              P.test_single_key, P.test_causal_row0_is_v0, P.test_two_keys_sigmoid,
              P.test_key_shift_invariance, P.test_joint_key_permutation_invariance_noncausal,
              lambda: P.test_transposed_flow_matches(True),
              lambda: P.test_transposed_flow_matches(False),
              P.test_gqa_equals_mha_on_repeated_kv, P.test_mla_equals_general_attention_on_v_copy,
              P.test_blocksparse_all_causal_blocks_equals_dense,
              lambda: P.test_split_combine_equals_unsplit(3, True),
              lambda: P.test_split_combine_equals_unsplit(7, False),
              P.test_split_bounds_cover_keys_once, P.test_split_with_empty_trailing_split]
    return calls


def _some_pin_fails():
    for pin in _pins():
        try:
            pin()
        except Exception:
            return True
    return False


def _orig(name):
    return getattr(A, name)


MUTANTS = {
    # GQA map with the wrong grouping (interleaved instead of contiguous groups)
    "gqa_interleaved": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    # scale dropped from the scores
    "no_scale": ("_scores", lambda q, k, scale: q @ k.T),
    # sign error in the scores
    "neg_scores": ("_scores", lambda q, k, scale: -scale * (q @ k.T)),
    # causal boundary off by one (strict) and top-left instead of bottom-right alignment
    "causal_strict": ("_causal_visible",
                      lambda rows, lq, lk: np.arange(lk)[None, :] < rows[:, None] + (lk - lq)),
    "causal_top_left": ("_causal_visible",
                        lambda rows, lq, lk: np.arange(lk)[None, :] <= rows[:, None]),
    # LSE in log2 / without the max term
    "lse_log2": ("_lse", lambda m, l: np.where(np.isfinite(m), m + np.log2(np.where(l > 0, l, 1)),
                                               -np.inf)),
    "lse_no_max": ("_lse", lambda m, l: np.where(np.isfinite(m), np.log(np.where(l > 0, l, 1)),
                                                 -np.inf)),
    # values contracted with the keys reversed (wrong index)
    "values_reversed": ("_weighted_values", lambda p, v: p @ v[::-1]),
    # block union replaced by intersection
    "sparse_intersection": ("blocksparse_row_mask", None),
    # split chunks overlapping by one key
    "split_overlap": ("split_bounds", None),
    # combine without normalising by the weight sum
    "combine_unnormalised": ("combine_lse", None),
}


def _sparse_intersection(rows, lk, blocks_of_qb, cols, block_m=64, block_n=64):
    rows = np.asarray(rows)
    nkb = -(-lk // block_n)
    colmask = np.zeros(lk, bool)
    if len(cols):
        colmask[np.asarray(cols)] = True
    out = np.zeros((rows.size, lk), bool)
    for qb in np.unique(rows // block_m):
        bm = np.zeros(nkb, bool)
        blk = np.asarray(blocks_of_qb(int(qb)), int)
        if blk.size:
            bm[blk] = True
        out[(rows // block_m) == qb] = np.repeat(bm, block_n)[:lk] & colmask
    return out


def _split_overlap(lk, s):
    per = -(-lk // s)
    c = 64 * (-(-per // 64))
    return [(max(0, min(i * c, lk) - 1), min((i + 1) * c, lk)) for i in range(s)]


def _combine_unnormalised(o_part, lse_part):
    o_part = np.asarray(o_part, float)
    lse_part = np.asarray(lse_part, float)
    mx = lse_part.max(axis=0)
    ok = np.isfinite(mx)
    safe = np.where(ok, mx, 0.0)
    w = np.where(ok[None], np.exp(lse_part - safe[None]), 0.0)
    o = (w[..., None] * o_part).sum(axis=0)
    lse = np.where(ok, mx + np.log(np.where(ok, w.sum(axis=0), 1.0)), -np.inf)
    return o, lse


_IMPL = {"sparse_intersection": _sparse_intersection, "split_overlap": _split_overlap,
         "combine_unnormalised": _combine_unnormalised}


def test_unmutated_oracle_passes_every_pin():
    for pin in _pins():
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(A, attr, fn if fn is not None else _IMPL[name])
    assert _some_pin_fails(), f"mutant {name} passed every pin"

"""Pins of the fp64 oracle against things other than itself (CPU only).

* brute force: pure-Python scalar loops (oracle/bruteforce.py) on tiny shapes;
* hand-derived golden values (tests/golden/hand_cases.json), worked out on paper;
* closed forms: uniform keys give (prefix) means, constant V gives that constant, one key gives
  that key's value, causal row 0 gives V_0, two keys give a sigmoid mix;
* invariants: shifting every key by one vector shifts LSE by scale*q.c and leaves O alone;
  permuting (K, V) jointly leaves non-causal O alone; the transposed flow of the FlashMLA-ETAP
  page ("Mecanismo Central") gives the same O;
* reductions: GQA == MHA on repeated K/V; MLA == general attention on an explicit V copy;
  block-sparse naming every causal block == dense causal; split + combine == unsplit.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle.bruteforce import attention_bruteforce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _f(x):
    """JSON value -> numpy array, with the strings "-inf"/"inf" as floats."""
    if isinstance(x, list):
        return np.array([_f(e) for e in x], dtype=np.float64)
    if isinstance(x, str):
        return float(x)
    return float(x)


def _golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _assert_close(a, b, tol):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        diff = np.where(both_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(diff)), "non-finite mismatch"
    assert diff.max(initial=0.0) <= tol, f"max diff {diff.max()} > {tol}"


# ----------------------------------------------------------------------------- golden
@pytest.mark.parametrize("case", _golden()["cases"], ids=lambda c: c["name"])
def test_golden_dense(case):
    q, k, v = _f(case["q"]), _f(case["k"]), _f(case["v"])
    o, lse = A.attention(q, k, v, case["scale"], case["causal"])
    _assert_close(o, _f(case["o"]), 1e-12)
    _assert_close(lse, _f(case["lse"]), 1e-12)


@pytest.mark.parametrize("case", _golden()["blocksparse_cases"], ids=lambda c: c["name"])
def test_golden_blocksparse(case):
    q, k, v = _f(case["q"]), _f(case["k"]), _f(case["v"])
    bs = case["block"]
    lq, lk = q.shape[1], k.shape[1]
    fn = A.csr_allowed_fn(case["blk_ptr"], case["blk_idx"], case["col_ptr"], case["col_idx"],
                          hq=q.shape[2], nqb=-(-lq // bs), lk=lk, block_m=bs, block_n=bs)
    o, lse = A.attention(q, k, v, case["scale"], case["causal"], allowed_fn=fn)
    _assert_close(o, _f(case["o"]), 1e-12)
    _assert_close(lse, _f(case["lse"]), 1e-12)


@pytest.mark.parametrize("case", _golden()["combine_cases"], ids=lambda c: c["name"])
def test_golden_combine(case):
    o, lse = A.combine_lse(_f(case["o_part"]), _f(case["lse_part"]))
    _assert_close(o, _f(case["o"]), 1e-12)
    _assert_close(lse, _f(case["lse"]), 1e-12)


# ----------------------------------------------------------------------------- brute force
BF_CASES = [
    # B, Hq, Hkv, Lq, Lk, Dqk, Dv, causal
    (1, 1, 1, 5, 5, 3, 3, True),
    (2, 4, 2, 6, 6, 4, 2, True),
    (1, 4, 1, 3, 7, 5, 4, True),     # Lq < Lk, bottom-right causal
    (2, 2, 2, 7, 4, 3, 3, False),    # Lq > Lk non-causal
    (1, 4, 4, 1, 9, 8, 8, False),    # decode shape
    (1, 2, 1, 1, 9, 6, 4, True),     # decode with causal: sees every key
]


@pytest.mark.parametrize("cfg", BF_CASES)
def test_bruteforce_dense(cfg):
    B, Hq, Hkv, Lq, Lk, Dqk, Dv, causal = cfg
    q = _rand((B, Lq, Hq, Dqk), 1)
    k = _rand((B, Lk, Hkv, Dqk), 2)
    v = _rand((B, Lk, Hkv, Dv), 3)
    scale = 0.7
    o, lse = A.attention(q, k, v, scale, causal)
    ob, lb = attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    _assert_close(o, ob, 1e-12)
    _assert_close(lse, lb, 1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bruteforce_blocksparse(seed):
    rng = np.random.default_rng(100 + seed)
    B, Hq, Hkv, L, D, bs = 1, 2, 1, 12, 3, 3
    q = _rand((B, L, Hq, D), 10 + seed)
    k = _rand((B, L, Hkv, D), 20 + seed)
    v = _rand((B, L, Hkv, D), 30 + seed)
    nqb = L // bs
    ptr, idx, cptr, cidx = [0], [], [0], []
    blocks = {}
    cols = {}
    for h in range(Hq):
        for qb in range(nqb):
            ids = sorted(set(rng.integers(0, nqb, size=rng.integers(0, 3)).tolist()))
            blocks[(h, qb)] = set(ids)
            idx += ids
            ptr.append(len(idx))
        cs = sorted(set(rng.integers(0, L, size=3).tolist()))
        cols[h] = set(cs)
        cidx += cs
        cptr.append(len(cidx))
    fn = A.csr_allowed_fn(ptr, idx, cptr, cidx, hq=Hq, nqb=nqb, lk=L, block_m=bs, block_n=bs)
    o, lse = A.attention(q, k, v, 0.9, True, allowed_fn=fn)
    vis = lambda b, h, i, j: (j // bs in blocks[(h, i // bs)]) or (j in cols[h])
    ob, lb = attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), 0.9, True, vis)
    _assert_close(o, ob, 1e-12)
    _assert_close(lse, lb, 1e-12)


# ----------------------------------------------------------------------------- closed forms
def test_uniform_keys_give_prefix_means():
    B, H, L, D = 1, 2, 37, 5
    q = _rand((B, L, H, D), 4)
    krow = _rand((D,), 5)
    k = np.broadcast_to(krow, (B, L, H, D)).copy()
    v = _rand((B, L, H, D), 6)
    scale = 0.3
    o, lse = A.attention(q, k, v, scale, True)
    csum = np.cumsum(v, axis=1)
    n = np.arange(1, L + 1)
    _assert_close(o, csum / n[None, :, None, None], 1e-12)
    s = scale * np.einsum("blhd,d->bhl", q, krow)
    _assert_close(lse, s + np.log(n)[None, None, :], 1e-12)


def test_constant_values_give_constant_output():
    q = _rand((2, 9, 4, 6), 7, 3.0)
    k = _rand((2, 11, 2, 6), 8, 3.0)
    v = np.full((2, 11, 2, 3), -1.75)
    o, _ = A.attention(q, k, v, 0.5, True)
    _assert_close(o, np.full(o.shape, -1.75), 1e-12)


def test_single_key():
    q = _rand((1, 1, 3, 4), 9)
    k = _rand((1, 1, 3, 4), 10)
    v = _rand((1, 1, 3, 2), 11)
    o, lse = A.attention(q, k, v, 0.25, False)
    _assert_close(o, v, 0.0)
    _assert_close(lse[0, :, 0], 0.25 * np.sum(q[0, 0] * k[0, 0], axis=-1), 1e-15)


def test_causal_row0_is_v0():
    q = _rand((1, 8, 2, 4), 12)
    k = _rand((1, 8, 2, 4), 13)
    v = _rand((1, 8, 2, 4), 14)
    o, lse = A.attention(q, k, v, 0.5, True)
    _assert_close(o[:, 0], v[:, 0], 0.0)
    _assert_close(lse[:, :, 0], 0.5 * np.sum(q[0, 0] * k[0, 0], axis=-1)[None], 1e-15)


def test_two_keys_sigmoid():
    q = _rand((1, 4, 1, 3), 15)
    k = _rand((1, 2, 1, 3), 16)
    v = _rand((1, 2, 1, 5), 17)
    o, lse = A.attention(q, k, v, 1.1, False)
    s0 = 1.1 * q[0, :, 0] @ k[0, 0, 0]
    s1 = 1.1 * q[0, :, 0] @ k[0, 1, 0]
    sig = 1.0 / (1.0 + np.exp(-(s0 - s1)))
    exp_o = sig[:, None] * v[0, 0, 0][None] + (1 - sig)[:, None] * v[0, 1, 0][None]
    _assert_close(o[0, :, 0], exp_o, 1e-14)
    _assert_close(lse[0, 0], np.logaddexp(s0, s1), 1e-14)


# ----------------------------------------------------------------------------- invariants
def test_key_shift_invariance():
    q = _rand((1, 6, 2, 4), 18)
    k = _rand((1, 6, 2, 4), 19)
    v = _rand((1, 6, 2, 4), 20)
    c = _rand((4,), 21)
    o1, l1 = A.attention(q, k, v, 0.6, True)
    o2, l2 = A.attention(q, k + c, v, 0.6, True)
    _assert_close(o1, o2, 1e-12)
    shift = 0.6 * np.einsum("blhd,d->bhl", q, c)
    _assert_close(l2, l1 + shift, 1e-12)


def test_joint_key_permutation_invariance_noncausal():
    q = _rand((1, 5, 2, 4), 22)
    k = _rand((1, 9, 1, 4), 23)
    v = _rand((1, 9, 1, 3), 24)
    perm = np.random.default_rng(25).permutation(9)
    o1, l1 = A.attention(q, k, v, 0.8, False)
    o2, l2 = A.attention(q, k[:, perm], v[:, perm], 0.8, False)
    _assert_close(o1, o2, 1e-12)
    _assert_close(l1, l2, 1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_transposed_flow_matches(causal):
    q = _rand((2, 7, 4, 5), 26)
    k = _rand((2, 10, 2, 5), 27)
    v = _rand((2, 10, 2, 3), 28)
    o1, _ = A.attention(q, k, v, 0.4, causal)
    o2 = A.attention_transposed(q, k, v, 0.4, causal)
    _assert_close(o1, o2, 1e-12)


def test_softmax_rows_sum_to_one_and_empty_rows_are_zero():
    s = _rand((6, 40), 43, 5.0)
    s[1, ::3] = -np.inf
    s[4, :] = -np.inf                       # no visible key
    p, m, l = A._softmax_rows(s)
    rs = p.sum(axis=1)
    _assert_close(np.delete(rs, 4), np.ones(5), 1e-13)
    assert rs[4] == 0.0 and np.isneginf(m[4]) and l[4] == 0.0
    assert np.all(p[1, ::3] == 0.0)


# ----------------------------------------------------------------------------- reductions
def test_gqa_equals_mha_on_repeated_kv():
    B, Hq, Hkv, L, D = 2, 8, 2, 6, 4
    q = _rand((B, L, Hq, D), 29)
    k = _rand((B, L, Hkv, D), 30)
    v = _rand((B, L, Hkv, D), 31)
    o1, l1 = A.attention(q, k, v, 0.5, True)
    g = Hq // Hkv
    o2, l2 = A.attention(q, np.repeat(k, g, axis=2), np.repeat(v, g, axis=2), 0.5, True)
    _assert_close(o1, o2, 1e-12)
    _assert_close(l1, l2, 1e-12)


def test_mla_equals_general_attention_on_v_copy():
    B, Hq, L, Dqk, Dv = 1, 4, 9, 12, 8
    q = _rand((B, 1, Hq, Dqk), 32)
    kl = _rand((B, L, 1, Dqk), 33)
    v = A.mla_value_view(kl, Dv)
    assert v.shape == (B, L, 1, Dv) and not np.shares_memory(v, kl)
    o, lse = A.attention(q, kl, v, 0.3, False)
    ob, lb = attention_bruteforce(q.tolist(), kl.tolist(), kl[..., :Dv].tolist(), 0.3, False)
    _assert_close(o, ob, 1e-12)
    _assert_close(lse, lb, 1e-12)


def test_blocksparse_all_causal_blocks_equals_dense():
    from workloads import dense_causal_lists
    B, Hq, Hkv, L, D = 1, 2, 1, 200, 4   # ragged: 200 = 3*64 + 8
    q = _rand((B, L, Hq, D), 34)
    k = _rand((B, L, Hkv, D), 35)
    v = _rand((B, L, Hkv, D), 36)
    ptr, idx, cptr, cidx = dense_causal_lists(B, Hq, L, L)
    fn = A.csr_allowed_fn(ptr, idx, cptr, cidx, hq=Hq, nqb=-(-L // 64), lk=L)
    o1, l1 = A.attention(q, k, v, 0.5, True, allowed_fn=fn)
    o2, l2 = A.attention(q, k, v, 0.5, True)
    _assert_close(o1, o2, 1e-12)
    _assert_close(l1, l2, 1e-12)


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 7])
@pytest.mark.parametrize("causal", [False, True])
def test_split_combine_equals_unsplit(splits, causal):
    B, Hq, Hkv, Lq, Lk, D = 1, 4, 2, 3, 300, 4
    q = _rand((B, Lq, Hq, D), 37)
    k = _rand((B, Lk, Hkv, D), 38)
    v = _rand((B, Lk, Hkv, D), 39)
    o1, l1 = A.attention(q, k, v, 0.5, causal)
    o2, l2 = A.attention_splitkv(q, k, v, 0.5, causal, splits)
    _assert_close(o1, o2, 1e-12)
    _assert_close(l1, l2, 1e-12)


def test_split_bounds_cover_keys_once():
    for lk in [1, 63, 64, 65, 300, 4096, 65536]:
        for s in [1, 2, 3, 5, 8, 32, 64]:
            if s > -(-lk // 64):
                continue
            b = A.split_bounds(lk, s)
            covered = np.zeros(lk, int)
            for lo, hi in b:
                assert lo % 64 == 0
                covered[lo:hi] += 1
            assert np.all(covered == 1)


def test_split_with_empty_trailing_split():
    # Lk = 130, S = 3: C = 64*ceil(44/64) = 64 -> ranges [0,64) [64,128) [128,130); S = 2 also
    # works; Lk = 65, S = 2: C = 64 -> [0,64) [64,65). Lk = 64*3, S = 3 with chunk 64.
    # Lk = 129, S = 3: per = 43 -> C = 64 -> [0,64) [64,128) [128,129): none empty; Lk = 150,
    # S = 3 -> per 50 -> C = 64 -> third split [128,150). Force an empty split: Lk = 256, S = 3:
    # per = 86 -> C = 128 -> [0,128) [128,256) [256,256) empty.
    assert A.split_bounds(256, 3)[2] == (256, 256)
    q = _rand((1, 2, 2, 4), 40)
    k = _rand((1, 256, 1, 4), 41)
    v = _rand((1, 256, 1, 4), 42)
    op, lp = A.splitkv_partials(q, k, v, 0.5, False, 3)
    assert np.all(np.isneginf(lp[2])) and np.all(op[2] == 0)
    o1, l1 = A.attention(q, k, v, 0.5, False)
    o2, l2 = A.attention_splitkv(q, k, v, 0.5, False, 3)
    _assert_close(o1, o2, 1e-12)
    _assert_close(l1, l2, 1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gathered_keys_equal_dense_mask(seed):
    """The gather form (scores over the listed keys only) equals the dense-mask form on random
    lists, causal, with Lq < Lk."""
    rng = np.random.default_rng(300 + seed)
    Lq, Lk, D, bs = 150, 260, 8, 64
    q, k, v = _rand((Lq, D), 40 + seed), _rand((Lk, D), 50 + seed), _rand((Lk, D), 60 + seed)
    nkb = -(-Lk // bs)
    cols = np.unique(rng.integers(0, Lk, 12))
    for qb in range(-(-Lq // bs)):
        blocks = np.unique(rng.integers(0, nkb, 2))
        rows = np.arange(qb * bs, min((qb + 1) * bs, Lq))
        keys = A.blocksparse_keys(blocks, cols, Lk, bs)
        og, lg = A.attention_rows_over_keys(q[rows], rows, k, v, 0.6, keys, Lq, Lk, True)
        mask = A.blocksparse_row_mask(rows, Lk, lambda _: blocks, cols, bs, bs)
        od, ld = A.attention_query_rows(q[rows], k[None, :, None], v[None, :, None], 0.6, True,
                                        0, 0, rows, Lq, 1, mask)
        _assert_close(og, od, 1e-12)
        _assert_close(lg, ld, 1e-12)


def test_blocksparse_keys_union_counts_each_key_once():
    keys = A.blocksparse_keys([0, 2], [1, 5, 64, 130, 300], 200, 64)
    assert list(keys) == sorted(set(range(0, 64)) | set(range(128, 192)) | {64})

"""GPU parity of attn_build_sparse_index (the dynamic block / column list builder) against the
fp64 oracle in oracle/sparse_index.py, through the C ABI.

The lists are index work decided by floating point (a top-k of scores), and the kernel ranks in
fp32 what the oracle ranks in fp64. So each list is compared as a set: equal to the oracle's,
or, where the two differ, every swapped element must sit at a near-tie of the oracle's ranking,
which is the only place rounding can move a top-k: within TOPK_REL_TOL of the k-th value for
column and slash importances, within TOPK_BLOCK_TOL of 1 + |k-th| for block scores, and within
TOPK_RANK_SLACK places of the k-th in the oracle's order (tests/helpers.py). The block
offsets (blk_ptr, col_ptr) are closed-form and compared exactly, and the list order (ascending)
is checked as is.
"""

import numpy as np
import pytest

from oracle import attention as A
from oracle import sparse_index as X
from tests.helpers import (TOPK_BLOCK_TOL, TOPK_RANK_SLACK, TOPK_REL_TOL, check_parity, say,
                           to_f64)
from workloads import WORKLOADS, make_qkv, randn_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _build(q, k, topk, ncols, scale):
    import torch
    import sparse_attention_attn_amd as S
    out = S.attn_build_sparse_index(q.to(DEV), k.to(DEV), topk, ncols, scale=scale)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def _check_topk_set(got, ref, scores, k_sel, forced, label, relative=True):
    """got / ref: ascending id arrays; scores: oracle scores over all ids (-inf for ids that
    cannot be listed); k_sel: ids picked besides the forced ones. relative: the band is
    TOPK_REL_TOL of the k-th score (column and slash importances) rather than TOPK_BLOCK_TOL of
    1 + |k-th| (block scores)."""
    assert np.all(np.diff(got) > 0), f"{label}: list not strictly ascending: {got}"
    if np.array_equal(got, ref):
        return
    assert got.size == ref.size, f"{label}: {got.size} ids, oracle {ref.size}"
    cand = [i for i in ref if i not in forced]
    kth = min(scores[i] for i in cand) if cand else np.inf
    tol = TOPK_REL_TOL * abs(kth) if relative else TOPK_BLOCK_TOL * (1.0 + abs(kth))
    diff = sorted(set(got) ^ set(ref))
    assert len(diff) <= 2 * TOPK_RANK_SLACK, f"{label}: {len(diff)} ids differ from the oracle's"
    ids = np.array([i for i in range(len(scores)) if i not in forced and np.isfinite(scores[i])])
    sc = np.asarray(scores, np.float64)[ids]
    order = ids[np.lexsort((ids, -sc))]           # the oracle's ranking: score, then lower id
    rank = {int(i): r for r, i in enumerate(order)}
    for i in diff:
        assert abs(scores[i] - kth) <= tol, (
            f"{label}: id {i} (score {scores[i]:.9g}) differs from the oracle's choice away from "
            f"a near-tie (k-th score {kth:.9g}, band {tol:.3g})")
        assert abs(rank[i] - (k_sel - 1)) <= TOPK_RANK_SLACK, (
            f"{label}: id {i} has oracle rank {rank[i] + 1}, not near {k_sel}")


def _compare(q, k, topk, ncols, scale, label):
    B, L, Hq, D = q.shape
    nqb = -(-L // 64)
    bp, bi, cp, ci = _build(q, k, topk, ncols, scale)
    rbp, rbi, rcp, rci, scores, imp = X.build_index(to_f64(q), to_f64(k), float(np.float32(scale)),
                                                     topk, ncols)
    assert np.array_equal(bp, rbp), f"{label}: blk_ptr"
    assert np.array_equal(cp, rcp), f"{label}: col_ptr"
    for b in range(B):
        for h in range(Hq):
            for qb in range(nqb):
                r = (b * Hq + h) * nqb + qb
                _check_topk_set(bi[bp[r]:bp[r + 1]], rbi[rbp[r]:rbp[r + 1]], scores[b, h, qb],
                                topk - 1, {qb}, f"{label} b={b} h={h} qb={qb}", relative=False)
            r = b * Hq + h
            _check_topk_set(ci[cp[r]:cp[r + 1]], rci[rcp[r]:rcp[r + 1]], imp[b, h], ncols, set(),
                            f"{label} columns b={b} h={h}")
    return bp, bi, cp, ci


SHAPES = [
    # B, Hq, Hkv, L, D, topk, ncols
    (1, 4, 2, 64, 128, 4, 10),        # one query block
    (2, 4, 2, 200, 128, 2, 30),       # ragged last block, GQA
    (1, 2, 1, 1000, 64, 5, 100),      # D = 64
    (1, 4, 4, 2049, 128, 40, 5000),   # more columns than keys: all keys listed
    (1, 8, 2, 3000, 128, 1, 0),       # diagonal only, no columns
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_build_index_matches_oracle(shape):
    B, Hq, Hkv, L, D, topk, ncols = shape
    say(f"sparse index {shape}")
    q = randn_bf16((B, L, Hq, D), 9100 + L)
    k = randn_bf16((B, L, Hkv, D), 9101 + L)
    _compare(q, k, topk, ncols, D ** -0.5, f"index{shape}")


def test_build_index_planted_structure():
    """Planted key blocks and columns that the estimator must find (far from any tie)."""
    B, Hq, Hkv, L, D = 1, 2, 1, 1024, 128
    say("sparse index planted")
    q = randn_bf16((B, L, Hq, D), 9200).float()
    k = randn_bf16((B, L, Hkv, D), 9201).float() * 0.2
    qm = q[0, 15 * 64:16 * 64, 0].mean(0)
    k[0, 3 * 64:4 * 64, 0] = 8.0 * qm / qm.norm()          # block 3 for query block 15 of head 0
    pm = q[0, L - 64:, 1].mean(0)
    k[0, 500, 0] = 40.0 * pm / pm.dot(pm)                  # column 500 for head 1's probe
    q, k = q.bfloat16(), k.bfloat16()
    bp, bi, cp, ci = _compare(q, k, 2, 5, D ** -0.5, "planted")
    assert list(bi[bp[15]:bp[16]]) == [3, 15]
    assert 500 in list(ci[cp[1]:cp[2]])


def test_build_index_deterministic():
    say("sparse index determinism")
    q = randn_bf16((1, 3000, 8, 128), 9300)
    k = randn_bf16((1, 3000, 2, 128), 9301)
    a = _build(q, k, 16, 200, 0.09)
    b = _build(q, k, 16, 200, 0.09)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_built_lists_drive_blocksparse_forward():
    """The builder's lists, fed to attn_fwd_blocksparse, give the oracle's attention over the
    same lists."""
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, L, D = 1, 4, 2, 1500, 128
    say("sparse index -> blocksparse forward")
    q = randn_bf16((B, L, Hq, D), 9400)
    k = randn_bf16((B, L, Hkv, D), 9401)
    v = randn_bf16((B, L, Hkv, D), 9402)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lists = S.attn_build_sparse_index(qd, kd, 6, 50, scale=D ** -0.5)
    o = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    S.attn_fwd_blocksparse(qd, kd, vd, o, *lists, lse=lse, causal=True, scale=D ** -0.5)
    torch.cuda.synchronize()
    bp, bi, cp, ci = [t.cpu().numpy() for t in lists]
    S.attn_blocksparse_check(bp, bi, cp, ci, B, Hq, L, L)
    allowed = A.csr_allowed_fn(bp, bi, cp, ci, Hq, -(-L // 64), L)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5),
                                 True, allowed_fn=allowed)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, "index->blocksparse")


def test_build_index_full_size_sampled():
    """The 128K block-sparse workload's shape (B 1, Hq 32, Hkv 8, L 131072, D 128), 96 blocks
    per query block and 1000 columns per head: two heads checked against the oracle, every
    query block of them plus their column lists."""
    w = WORKLOADS["blocksparse_128k"]
    say(f"sparse index full size {w.name}")
    q, k, _ = make_qkv(w)
    topk, ncols = 96, 1000
    bp, bi, cp, ci = _build(q, k, topk, ncols, w.scale)
    nqb = -(-w.Lq // 64)
    sc = float(np.float32(w.scale))
    for h in (0, 29):
        qh = q[0, :, h].double().numpy()
        kh = k[0, :, h // (w.Hq // w.Hkv)].double().numpy()
        scores = X.block_scores(qh, kh, sc, 64)
        for qb in range(nqb):
            r = h * nqb + qb
            ref = X.select_blocks(scores[qb], qb, topk)
            _check_topk_set(bi[bp[r]:bp[r + 1]], ref, scores[qb], topk - 1, {qb},
                            f"full h={h} qb={qb}", relative=False)
        imp = X.probe_importance(qh, kh, sc, 64)
        _check_topk_set(ci[cp[h]:cp[h + 1]], X.select_columns(imp, ncols), imp, ncols, set(),
                        f"full columns h={h}")


def test_build_index_exact_ties_take_lowest_ids():
    """Every key row equal: the pooled block scores are bitwise equal (the sums of equal bf16
    values are exact in fp32), so the lists are exact ties, broken toward the lowest ids. The
    probe importance is flat over the keys every probe row sees, so the column list is the
    lowest indices."""
    import torch
    B, Hq, Hkv, L, D, topk, ncols = 1, 4, 2, 1000, 128, 5, 40
    say("sparse index exact ties")
    q = randn_bf16((B, L, Hq, D), 9500)
    k = randn_bf16((1, 1, Hkv, D), 9501).expand(B, L, Hkv, D).contiguous()
    bp, bi, cp, ci = _build(q, k, topk, ncols, D ** -0.5)
    rbp, rbi, rcp, rci, _, _ = X.build_index(to_f64(q), to_f64(k), float(np.float32(D ** -0.5)),
                                             topk, ncols)
    assert np.array_equal(bp, rbp) and np.array_equal(bi, rbi)
    assert np.array_equal(cp, rcp) and np.array_equal(ci, rci)
    nqb = -(-L // 64)
    for h in range(Hq):
        for qb in range(nqb):
            r = h * nqb + qb
            assert list(bi[bp[r]:bp[r + 1]]) == sorted(set(range(min(topk - 1, qb))) | {qb})
        assert list(ci[cp[h]:cp[h + 1]]) == list(range(ncols))


def test_build_index_negative_scale():
    """A negative scale reverses the ranking of the block scores and of the probe scores."""
    say("sparse index negative scale")
    q = randn_bf16((1, 1500, 4, 128), 9600)
    k = randn_bf16((1, 1500, 2, 128), 9601)
    _compare(q, k, 6, 80, -0.08, "negative scale")


# ---- vertical-slash lists (attn_build_vslash_index) -----------------------------------------
def _build_vs(q, k, ncols, nslash, scale):
    import torch
    import sparse_attention_attn_amd as S
    out = S.attn_build_vslash_index(q.to(DEV), k.to(DEV), ncols, nslash, scale=scale)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def _compare_vs(q, k, ncols, nslash, scale, label):
    B, L, Hq, D = q.shape
    cp, ci, sp, si = _build_vs(q, k, ncols, nslash, scale)
    rcp, rci, rsp, rsi, cimp, simp = X.build_vslash_index(to_f64(q), to_f64(k),
                                                          float(np.float32(scale)), ncols, nslash)
    assert np.array_equal(cp, rcp) and np.array_equal(sp, rsp), f"{label}: pointers"
    for r in range(B * Hq):
        b, h = divmod(r, Hq)
        _check_topk_set(ci[cp[r]:cp[r + 1]], rci[rcp[r]:rcp[r + 1]], cimp[b, h], ncols, set(),
                        f"{label} columns b={b} h={h}")
        _check_topk_set(si[sp[r]:sp[r + 1]], rsi[rsp[r]:rsp[r + 1]], simp[b, h], nslash, set(),
                        f"{label} slashes b={b} h={h}")
    return cp, ci, sp, si


VS_SHAPES = [
    # B, Hq, Hkv, L, D, ncols, nslash
    (1, 4, 2, 64, 128, 10, 10),
    (2, 4, 2, 200, 128, 30, 40),
    (1, 2, 1, 1000, 64, 100, 70),
    (1, 4, 4, 2049, 128, 5000, 3000),   # more than L: everything listed
    (1, 8, 2, 3000, 128, 0, 25),
    (1, 2, 2, 40, 128, 7, 7),           # L < 64: every row probes
]


@pytest.mark.parametrize("shape", VS_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_build_vslash_index_matches_oracle(shape):
    B, Hq, Hkv, L, D, ncols, nslash = shape
    say(f"vslash index {shape}")
    q = randn_bf16((B, L, Hq, D), 9700 + L)
    k = randn_bf16((B, L, Hkv, D), 9701 + L)
    _compare_vs(q, k, ncols, nslash, D ** -0.5, f"vs{shape}")


def test_build_vslash_index_planted_diagonal():
    B, Hq, Hkv, L, D, ostar = 1, 2, 1, 1500, 128, 333
    say("vslash index planted diagonal")
    q = randn_bf16((B, L, Hq, D), 9800).float()
    k = randn_bf16((B, L, Hkv, D), 9801).float() * 0.1
    for r in range(L - 64, L):
        qr = q[0, r, 0]
        k[0, r - ostar, 0] = 60.0 * qr / qr.dot(qr)
    q, k = q.bfloat16(), k.bfloat16()
    cp, ci, sp, si = _compare_vs(q, k, 20, 5, D ** -0.5, "planted diagonal")
    assert ostar in list(si[sp[0]:sp[1]])


def test_built_vslash_lists_drive_forward():
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, L, D = 1, 4, 2, 1300, 128
    say("vslash index -> vertical-slash forward")
    q = randn_bf16((B, L, Hq, D), 9900)
    k = randn_bf16((B, L, Hkv, D), 9901)
    v = randn_bf16((B, L, Hkv, D), 9902)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    cp, ci, sp, si = S.attn_build_vslash_index(qd, kd, 60, 90, scale=D ** -0.5)
    nqb = -(-L // 64)
    bp = torch.zeros(B * Hq * nqb + 1, dtype=torch.int32, device=DEV)
    bi = torch.zeros(1, dtype=torch.int32, device=DEV)
    o = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    S.attn_fwd_vertical_slash(qd, kd, vd, o, bp, bi, cp, ci, sp, si, lse=lse, scale=D ** -0.5)
    torch.cuda.synchronize()
    hcp, hci, hsp, hsi = [t.cpu().numpy() for t in (cp, ci, sp, si)]
    S.attn_vertical_slash_check(hsp, hsi, B, Hq, L)
    fn = A.vslash_allowed_fn(np.zeros(B * Hq * nqb + 1, np.int32), np.zeros(0, np.int32), hcp,
                             hci, hsp, hsi, Hq, nqb, L, L)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5),
                                 True, allowed_fn=fn)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, "vslash index -> forward")


def test_build_vslash_index_full_size_sampled():
    """The 128K shape, 1000 columns and 1088 lines per head: two heads against the oracle."""
    w = WORKLOADS["vslash_128k"]
    say(f"vslash index full size {w.name}")
    q, k, _ = make_qkv(w)
    ncols, nslash = 1000, 1088
    cp, ci, sp, si = _build_vs(q, k, ncols, nslash, w.scale)
    sc = float(np.float32(w.scale))
    for h in (3, 30):
        qh = q[0, :, h].double().numpy()
        kh = k[0, :, h // (w.Hq // w.Hkv)].double().numpy()
        cimp = X.probe_importance(qh, kh, sc, 64)
        simp = X.slash_importance(qh, kh, sc, 64)
        _check_topk_set(ci[cp[h]:cp[h + 1]], X.select_columns(cimp, ncols), cimp, ncols, set(),
                        f"full columns h={h}")
        _check_topk_set(si[sp[h]:sp[h + 1]], X.select_columns(simp, nslash), simp, nslash, set(),
                        f"full slashes h={h}")


def test_build_vslash_index_deterministic():
    say("vslash index determinism")
    q = randn_bf16((1, 2500, 4, 128), 9950)
    k = randn_bf16((1, 2500, 2, 128), 9951)
    a = _build_vs(q, k, 100, 200, 0.09)
    b = _build_vs(q, k, 100, 200, 0.09)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_builders_on_structured_inputs():
    """Both builders on the structured inputs the bench uses for its dynamic pipelines
    (workloads.make_structured_qk: a planted band and planted columns), at 4096 tokens: the
    lists match the oracle's, and the planted band is what they find (the diagonal's
    neighbourhood among the blocks, the first offsets among the slash lines)."""
    from workloads import make_structured_qk
    B, Hq, Hkv, L, D = 1, 4, 2, 4096, 128
    say("index builders on structured inputs")
    q, k = make_structured_qk(B, L, Hq, Hkv, D, 9400, window=1024, n_cols=40, band_logit=12.0,
                              col_logit=5.0, device="cpu")
    bp, bi, cp, ci = _compare(q, k, 8, 60, D ** -0.5, "structured blocks")
    nqb = L // 64
    for h in range(Hq):
        for qb in range(8, nqb):
            row = bi[bp[h * nqb + qb]:bp[h * nqb + qb + 1]]
            assert np.all(row >= qb - 12), f"head {h} query block {qb}: {row}"
    cp, ci, sp, si = _compare_vs(q, k, 60, 300, D ** -0.5, "structured lines")
    for h in range(Hq):
        offs = si[sp[h]:sp[h + 1]]
        assert np.count_nonzero(offs < 400) >= 280, f"head {h}: {offs}"

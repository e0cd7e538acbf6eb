"""GPU parity of attn_fwd_blocksparse against the fp64 oracle (lists -> mask by np.repeat of a
block bitmap OR a column bitmap: no code shared with the kernel's walk/gather/de-dup)."""

import numpy as np
import pytest

from oracle import attention as A
from tests.helpers import check_parity, say, to_f64
from workloads import (WORKLOADS, dense_causal_lists, make_blocksparse_lists, make_qkv,
                       randn_bf16, sampled_rows)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(q, k, v, lists, causal, scale):
    import torch
    import sparse_attention_attn_amd as S
    B, Lq, Hq, _ = q.shape
    o = torch.empty((B, Lq, Hq, v.shape[3]), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    dl = [torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(DEV) for x in lists]
    S.attn_fwd_blocksparse(q, k, v, o, *dl, lse=lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _oracle(q, k, v, lists, causal, scale):
    B, Lq, Hq, _ = q.shape
    Lk = k.shape[1]
    fn = A.csr_allowed_fn(*lists, hq=Hq, nqb=-(-Lq // 64), lk=Lk)
    return A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(scale), causal,
                       allowed_fn=fn)


CASES = [
    # B, Hq, Hkv, L, D, local, p_extra, n_cols
    (1, 4, 2, 1000, 128, 4, 0.10, 50),
    (2, 4, 1, 777, 64, 3, 0.20, 120),
    (1, 8, 2, 2048, 128, 8, 0.05, 300),
    (1, 2, 2, 130, 128, 1, 0.00, 40),    # columns only (plus the diagonal)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_blocksparse_small(case):
    B, Hq, Hkv, L, D, local, p, ncols = case
    say(f"blocksparse {case}")
    seed = 9000 + sum(case[:5])
    q = randn_bf16((B, L, Hq, D), seed)
    k = randn_bf16((B, L, Hkv, D), seed + 1)
    v = randn_bf16((B, L, Hkv, D), seed + 2)
    lists = make_blocksparse_lists(B, Hq, L, L, seed + 3, local_blocks=local, p_extra=p,
                                   n_cols=ncols)
    import sparse_attention_attn_amd as S
    S.attn_blocksparse_check(*lists, B, Hq, L, L)
    o, lse = _run(q.to(DEV), k.to(DEV), v.to(DEV), lists, True, D ** -0.5)
    o_ref, lse_ref = _oracle(q, k, v, lists, True, D ** -0.5)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"sparse{case}")


def test_blocksparse_all_blocks_equals_dense():
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, L, D = 1, 4, 2, 700, 128
    say("blocksparse all blocks == dense causal")
    q, k, v = (randn_bf16((B, L, Hq, D), 9100), randn_bf16((B, L, Hkv, D), 9101),
               randn_bf16((B, L, Hkv, D), 9102))
    lists = dense_causal_lists(B, Hq, L, L)
    o, lse = _run(q.to(DEV), k.to(DEV), v.to(DEV), lists, True, D ** -0.5)
    od = torch.empty_like(o)
    ld = torch.empty_like(lse)
    S.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), od, ld, causal=True, scale=D ** -0.5)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5), True)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, "sparse-all")
    check_parity(to_f64(od), o_ref, to_f64(ld), lse_ref, "dense")


def test_blocksparse_noncausal_and_empty_rows():
    """Non-causal lists, a query block with no block and no column (O = 0, LSE = -inf)."""
    B, Hq, Hkv, L, D = 1, 2, 1, 256, 64
    say("blocksparse non-causal + empty rows")
    q, k, v = (randn_bf16((B, L, Hq, D), 9200), randn_bf16((B, L, Hkv, D), 9201),
               randn_bf16((B, L, Hkv, D), 9202))
    # head 0: qb0 -> {3}, qb1 -> {}, qb2 -> {0, 2}, qb3 -> {1, 3}; columns {5, 70}
    # head 1: every query block empty, no columns
    blk_ptr = np.array([0, 1, 1, 3, 5, 5, 5, 5, 5], np.int32)
    blk_idx = np.array([3, 0, 2, 1, 3], np.int32)
    col_ptr = np.array([0, 2, 2], np.int32)
    col_idx = np.array([5, 70], np.int32)
    lists = (blk_ptr, blk_idx, col_ptr, col_idx)
    o, lse = _run(q.to(DEV), k.to(DEV), v.to(DEV), lists, False, 0.125)
    o_ref, lse_ref = _oracle(q, k, v, lists, False, 0.125)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, "sparse-noncausal")
    assert np.all(np.isneginf(to_f64(lse)[0, 1]))


def test_planted_columns_counted_once():
    """Planted keys make each column carry a large weight: a column counted twice (it is also
    inside a listed block), a missed column, or a column past the causal horizon that leaks in
    would move O by far more than the tolerance."""
    import torch
    B, Hq, Hkv, L, D = 1, 1, 1, 512, 64
    say("planted columns")
    q = randn_bf16((B, L, Hq, D), 9300).float()
    k = randn_bf16((B, L, Hkv, D), 9301).float() * 0.05
    v = randn_bf16((B, L, Hkv, D), 9302).float()
    cols = [10, 100, 130, 300, 450]
    probe = q[0, 400, 0]
    for c in cols:
        k[0, c, 0] = probe * 0.5
        v[0, c, 0] = 2.0 + c / 300.0   # |O| < 4: output rounding stays far inside 1e-2
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    nqb = L // 64
    # qb 6 (rows 384..447) lists block 1 (keys 64..127, contains column 100) and its diagonal
    blk_ptr, blk_idx = [0], []
    for qb in range(nqb):
        ids = sorted({qb, 1} if qb >= 1 else {0})
        blk_idx += ids
        blk_ptr.append(len(blk_idx))
    lists = (np.array(blk_ptr, np.int32), np.array(blk_idx, np.int32),
             np.array([0, len(cols)], np.int32), np.array(cols, np.int32))
    o, lse = _run(q.to(DEV), k.to(DEV), v.to(DEV), lists, True, D ** -0.5)
    o_ref, lse_ref = _oracle(q, k, v, lists, True, D ** -0.5)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, "planted-cols")


@pytest.fixture(scope="module")
def sparse128k():
    """The 128K block-sparse workload at full size, run once (the launch the bench times):
    inputs, lists and the GPU output on 4096 sampled rows (rows 0-63, the last 64 rows and
    3968 seeded rows)."""
    w = WORKLOADS["blocksparse_128k"]
    say(f"blocksparse_128k full size {w}")
    q, k, v = make_qkv(w)
    lists = make_blocksparse_lists(w.B, w.Hq, w.Lq, w.Lk, 1000 * w.index + 3)
    o, lse = _run(q.to(DEV), k.to(DEV), v.to(DEV), lists, True, w.scale)
    rows = sampled_rows(w.Lq, 4096, 1000 * w.index + 4, edge=64)
    return (w, q, k, v, lists, rows, o[0, rows].float().cpu().numpy(),
            lse[0][:, rows].cpu().numpy())


@pytest.mark.parametrize("group", range(4), ids=lambda g: f"heads{8 * g}-{8 * g + 7}")
def test_blocksparse_workload_full_size_sampled_rows(sparse128k, group):
    """The 4096 sampled rows of 8 query heads per case (all 32 over the four cases). The
    oracle scores each query block's sampled rows over that block's listed keys only
    (attention_rows_over_keys), which is the plain definition restricted to the keys the mask
    can leave visible."""
    w, q, k, v, (bp, bi, cp, ci), rows, of, lf = sparse128k
    nqb = w.Lq // 64
    g = w.Hq // w.Hkv
    sc = A.effective_scale(w.scale)
    qbs = rows // 64
    got_o, ref_o, got_l, ref_l = [], [], [], []
    for h in range(8 * group, 8 * group + 8):
        kh = k[0, :, h // g].double().numpy()
        vh = v[0, :, h // g].double().numpy()
        cols = ci[cp[h]:cp[h + 1]]
        for qb in np.unique(qbs):
            sel = qbs == qb
            rr = rows[sel]
            keys = A.blocksparse_keys(bi[bp[h * nqb + qb]:bp[h * nqb + qb + 1]], cols, w.Lk)
            orow, lrow = A.attention_rows_over_keys(q[0, rr, h].double().numpy(), rr, kh, vh, sc,
                                                    keys, w.Lq, w.Lk, True)
            got_o.append(of[sel, h])
            ref_o.append(orow)
            got_l.append(lf[h, sel])
            ref_l.append(lrow)
    check_parity(np.concatenate(got_o), np.concatenate(ref_o), np.concatenate(got_l),
                 np.concatenate(ref_l), f"sparse128k 4096 rows, heads {8 * group}-{8 * group + 7}",
                 record="blocksparse_128k")


def test_blocksparse_deterministic():
    B, Hq, Hkv, L, D = 1, 4, 2, 1500, 128
    say("determinism blocksparse")
    q, k, v = (randn_bf16((B, L, Hq, D), 9400), randn_bf16((B, L, Hkv, D), 9401),
               randn_bf16((B, L, Hkv, D), 9402))
    lists = make_blocksparse_lists(B, Hq, L, L, 9403, local_blocks=4, p_extra=0.1, n_cols=200)
    o1, l1 = _run(q.to(DEV), k.to(DEV), v.to(DEV), lists, True, D ** -0.5)
    o2, l2 = _run(q.to(DEV), k.to(DEV), v.to(DEV), lists, True, D ** -0.5)
    assert bool((o1 == o2).all()) and bool((l1 == l2).all())


def _jump_qkv(B, H, Hkv, L, D, seed):
    """Scores that rise by about 29 (exp2 domain) per 32 keys in KV head 0, fall in KV head 1
    and alternate in the others: weights against a reference set on earlier keys overflow fp32
    within a few units, so the kernel has to move its reference mid-row (its slow path)."""
    import torch
    u = torch.full((D,), 1.0)
    t = 20.0 * (torch.arange(L) // 32).float()
    q = u.expand(B, L, H, D) + 0.1 * randn_bf16((B, L, H, D), seed).float()
    k = 0.1 * randn_bf16((B, L, Hkv, D), seed + 1).float()
    k[:, :, 0] += t[:, None] / 8.0
    k[:, :, 1] += t.flip(0)[:, None] / 8.0
    for h in range(2, Hkv):
        k[:, :, h] += (t[:, None] / 8.0) * ((torch.arange(L) % 64) < 32).float()[:, None]
    # V halved (exact): peaked rows follow single value rows, and |O| < 4 keeps bf16 output
    # rounding below the 1e-2 bar
    v = 0.5 * randn_bf16((B, L, Hkv, D), seed + 2).float()
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


@pytest.mark.parametrize("D", [128, 64])
def test_blocksparse_reference_jumps(D):
    say(f"blocksparse reference jumps D={D}")
    B, Hq, Hkv, L = 1, 6, 3, 640
    q, k, v = _jump_qkv(B, Hq, Hkv, L, D, 9700 + D)
    lists = make_blocksparse_lists(B, Hq, L, L, 9710 + D, local_blocks=2, p_extra=0.4,
                                   n_cols=90)
    scale = D ** -0.5
    for causal in (True, False):
        o, lse = _run(q.to(DEV), k.to(DEV), v.to(DEV), lists, causal, scale)
        o_ref, lse_ref = _oracle(q, k, v, lists, causal, scale)
        assert np.isfinite(to_f64(o)).all()
        check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"sparse jumps causal={causal}")


def test_blocksparse_peaky():
    """Q x 4 (rounded to bf16): attention concentrated on few keys of the union."""
    import torch
    say("blocksparse peaky")
    B, Hq, Hkv, L, D = 1, 8, 2, 1500, 128
    q = (randn_bf16((B, L, Hq, D), 9800).float() * 4.0).to(torch.bfloat16)
    k = randn_bf16((B, L, Hkv, D), 9801)
    v = randn_bf16((B, L, Hkv, D), 9802) * 0.5  # |O| < 4 (see _jump_qkv)
    lists = make_blocksparse_lists(B, Hq, L, L, 9803, local_blocks=4, p_extra=0.1, n_cols=200)
    o, lse = _run(q.to(DEV), k.to(DEV), v.to(DEV), lists, True, D ** -0.5)
    o_ref, lse_ref = _oracle(q, k, v, lists, True, D ** -0.5)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, "sparse peaky")

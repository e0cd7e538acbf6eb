"""GPU parity of attn_fwd_vertical_slash (block/column union plus per-head slash lines)
against the fp64 oracle, through the C ABI.

Slash line o: query row i sees key i + (Lk - Lq) - o. Cases: slashes alone, slashes with
columns and blocks that overlap them (each key counted once), Lq < Lk alignment, D = 64,
non-causal blocks above the diagonal, every offset listed (= dense causal), empty slash lists
(bitwise equal to attn_fwd_blocksparse), determinism, and the 128K vertical-slash workload
on sampled rows.
"""

import numpy as np
import pytest

from oracle import attention as A
from tests.helpers import check_parity, say, to_f64
from workloads import (WORKLOADS, make_qkv, make_vslash_lists, randn_bf16, sampled_rows)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _csr(per_head_lists):
    ptr, parts = [0], []
    for x in per_head_lists:
        x = np.asarray(sorted(set(int(v) for v in x)), np.int32)
        parts.append(x)
        ptr.append(ptr[-1] + x.size)
    idx = np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)
    return np.asarray(ptr, np.int32), idx


def _dev(x):
    import torch
    return torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32)).to(DEV)


def _run(q, k, v, bp, bi, cp, ci, sp, si, causal=True, scale=None):
    import torch
    import sparse_attention_attn_amd as S
    B, Lq, Hq, D = q.shape
    scale = D ** -0.5 if scale is None else scale
    o = torch.empty((B, Lq, Hq, v.shape[3]), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    S.attn_fwd_vertical_slash(q.to(DEV), k.to(DEV), v.to(DEV), o, _dev(bp), _dev(bi), _dev(cp),
                              _dev(ci), _dev(sp), _dev(si), lse=lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _compare(q, k, v, bp, bi, cp, ci, sp, si, label, causal=True):
    B, Lq, Hq, D = q.shape
    Lk = k.shape[1]
    import sparse_attention_attn_amd as S
    S.attn_blocksparse_check(bp, bi, cp, ci, B, Hq, Lq, Lk)
    S.attn_vertical_slash_check(sp, si, B, Hq, Lk)
    o, lse = _run(q, k, v, bp, bi, cp, ci, sp, si, causal)
    fn = A.vslash_allowed_fn(bp, bi, cp, ci, sp, si, Hq, -(-Lq // 64), Lq, Lk)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5),
                                 causal, allowed_fn=fn)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, label)


def _no_blocks(B, Hq, Lq):
    return np.zeros(B * Hq * -(-Lq // 64) + 1, np.int32), np.zeros(0, np.int32)


def _qkv(B, Lq, Lk, Hq, Hkv, D, seed):
    return (randn_bf16((B, Lq, Hq, D), seed), randn_bf16((B, Lk, Hkv, D), seed + 1),
            randn_bf16((B, Lk, Hkv, D), seed + 2))


def test_slashes_only():
    B, Hq, Hkv, L, D = 1, 4, 2, 700, 128
    say("vslash: slashes only")
    q, k, v = _qkv(B, L, L, Hq, Hkv, D, 7000)
    rng = np.random.default_rng(1)
    sp, si = _csr([[0, 1, 2, 63, 64, 65, 127, 200] + rng.choice(np.arange(201, L), 10, False).tolist()
                   for _ in range(B * Hq)])
    bp, bi = _no_blocks(B, Hq, L)
    cp, ci = np.zeros(B * Hq + 1, np.int32), np.zeros(0, np.int32)
    _compare(q, k, v, bp, bi, cp, ci, sp, si, "slashes only")


def test_slashes_columns_blocks_overlap():
    """Slash keys that are also listed columns or inside listed blocks are counted once."""
    B, Hq, Hkv, L, D = 2, 4, 2, 777, 128
    say("vslash: union with overlaps")
    q, k, v = _qkv(B, L, L, Hq, Hkv, D, 7100)
    rng = np.random.default_rng(2)
    nqb = -(-L // 64)
    blocks = []
    for _ in range(B * Hq):
        for qb in range(nqb):
            blocks.append([0, qb] + rng.choice(np.arange(qb + 1), min(2, qb + 1), False).tolist())
    bp, bi = _csr(blocks)
    cp, ci = _csr([[0, 5, 64, 100, 300, 776] + rng.choice(L, 20, False).tolist()
                   for _ in range(B * Hq)])
    sp, si = _csr([list(range(0, 40)) + [64, 100, 128, 500] + rng.choice(L, 15, False).tolist()
                   for _ in range(B * Hq)])
    _compare(q, k, v, bp, bi, cp, ci, sp, si, "union overlap")


def test_wide_band_full_and_masked_tiles():
    """A band of 300 offsets: run tiles wholly inside it take the unmasked tile math, those that
    hold a listed column or cross the band's edges keep their masks; listed blocks inside the
    band and columns below every row (gathered tiles without a mask) are counted once."""
    B, Hq, Hkv, L, D = 1, 4, 2, 1500, 128
    say("vslash: wide band, full and masked tiles")
    q, k, v = _qkv(B, L, L, Hq, Hkv, D, 7150)
    rng = np.random.default_rng(5)
    nqb = -(-L // 64)
    bp, bi = _csr([[max(qb - 2, 0)] + ([1] if qb % 3 == 0 else []) for _ in range(B * Hq)
                   for qb in range(nqb)])
    cp, ci = _csr([list(range(0, 64)) + [130, 500, 501, 900, 1400] + rng.choice(L, 12, False).tolist()
                   for _ in range(B * Hq)])
    sp, si = _csr([list(range(0, 300)) + rng.choice(np.arange(300, L), 8, False).tolist()
                   for _ in range(B * Hq)])
    _compare(q, k, v, bp, bi, cp, ci, sp, si, "wide band")


def test_bottom_right_alignment_and_d64():
    B, Hq, Hkv, Lq, Lk, D = 1, 2, 1, 333, 1000, 64
    say("vslash: Lq < Lk, D 64")
    q, k, v = _qkv(B, Lq, Lk, Hq, Hkv, D, 7200)
    rng = np.random.default_rng(3)
    bp, bi = _no_blocks(B, Hq, Lq)
    cp, ci = _csr([rng.choice(Lk, 30, False) for _ in range(B * Hq)])
    sp, si = _csr([[0, 3, 17] + rng.choice(Lk, 25, False).tolist() for _ in range(B * Hq)])
    _compare(q, k, v, bp, bi, cp, ci, sp, si, "alignment d64")


@pytest.mark.parametrize("Lq,Lk,D", [(700, 700, 128), (300, 900, 128), (500, 260, 64)],
                         ids=["square", "lq_lt_lk", "lq_gt_lk_d64"])
def test_isolated_lines_planted(Lq, Lk, D):
    """Isolated slash lines (no neighbour offset listed: the per-wave window phase) beside a run
    of offsets (the tile phase). Keys on two isolated lines are planted so that each carries
    about half of its rows' weight (K row parallel to the row's Q, large V): a line missed, a
    pair counted twice, or a wrong key moves O by far more than the tolerance. Some planted keys
    are also listed columns or inside listed blocks (counted once), and with Lq > Lk the lines
    start at negative keys for the first rows. The planted keys dominate their rows (scores
    near 20 against about 1), so O there is close to 1; one row in three is planted, which keeps
    the mean |O| (and with it the mean-abs error of bf16 weights) near that of plain inputs."""
    import torch
    B, Hq, Hkv = 1, 4, 2
    say(f"vslash isolated lines Lq={Lq} Lk={Lk} D={D}")
    q, k, v = _qkv(B, Lq, Lk, Hq, Hkv, D, 7700 + Lq)
    off = Lk - Lq
    lines = [37, 211]                      # isolated offsets for every head
    run = list(range(0, 6))                # a run: tile phase
    kf, vf = k.float(), v.float()
    for h in range(Hkv):
        hq = h * (Hq // Hkv)               # plant for the first query head of each group
        for n, o in enumerate(lines):
            for i in range(3 * n, Lq, 6):  # rows 0 mod 6 on one line, 3 mod 6 on the other
                j = i + off - o
                if 0 <= j < Lk:
                    qi = q[0, i, hq].float()
                    kf[0, j, h] = 6.0 * qi / qi.norm() * (D ** 0.25)
                    vf[0, j, h] = 1.0
    k, v = kf.to(torch.bfloat16), vf.to(torch.bfloat16)
    nqb = -(-Lq // 64)
    bp, bi = _csr([[qb % max(1, -(-Lk // 64))] for _ in range(B * Hq) for qb in range(nqb)])
    cols = [[j for j in (5 + off - 37, 90 + off - 211, 301 + off - 37) if 0 <= j < Lk]
            for _ in range(B * Hq)]
    cp, ci = _csr(cols)
    sp, si = _csr([run + lines for _ in range(B * Hq)])
    _compare(q, k, v, bp, bi, cp, ci, sp, si, f"isolated lines {Lq}x{Lk}")


def test_noncausal_blocks_above_diagonal():
    B, Hq, Hkv, L, D = 1, 2, 2, 400, 128
    say("vslash: non-causal")
    q, k, v = _qkv(B, L, L, Hq, Hkv, D, 7300)
    nqb = -(-L // 64)
    bp, bi = _csr([[min(qb + 2, nqb - 1)] for _ in range(B * Hq) for qb in range(nqb)])
    cp, ci = _csr([[1, 399] for _ in range(B * Hq)])
    sp, si = _csr([[0, 9, 70] for _ in range(B * Hq)])
    _compare(q, k, v, bp, bi, cp, ci, sp, si, "non-causal", causal=False)


def test_every_offset_is_dense_causal():
    B, Hq, Hkv, L, D = 1, 2, 1, 300, 128
    say("vslash: every offset")
    q, k, v = _qkv(B, L, L, Hq, Hkv, D, 7400)
    bp, bi = _no_blocks(B, Hq, L)
    cp, ci = np.zeros(B * Hq + 1, np.int32), np.zeros(0, np.int32)
    sp, si = _csr([range(L) for _ in range(B * Hq)])
    o, lse = _run(q, k, v, bp, bi, cp, ci, sp, si)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5),
                                 True)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, "every offset")


def test_empty_slashes_equal_blocksparse_bitwise():
    import torch
    import sparse_attention_attn_amd as S
    from workloads import make_blocksparse_lists
    B, Hq, Hkv, L, D = 1, 4, 2, 1000, 128
    say("vslash: empty slash lists")
    q, k, v = _qkv(B, L, L, Hq, Hkv, D, 7500)
    bp, bi, cp, ci = make_blocksparse_lists(B, Hq, L, L, 7503, local_blocks=4, n_cols=50)
    sp, si = np.zeros(B * Hq + 1, np.int32), np.zeros(0, np.int32)
    o1, l1 = _run(q, k, v, bp, bi, cp, ci, sp, si)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    S.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), o2, _dev(bp), _dev(bi), _dev(cp),
                           _dev(ci), lse=l2, scale=D ** -0.5)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_deterministic():
    B, Hq, Hkv, L, D = 1, 2, 1, 500, 128
    say("vslash: determinism")
    q, k, v = _qkv(B, L, L, Hq, Hkv, D, 7600)
    bp, bi = _no_blocks(B, Hq, L)
    cp, ci = _csr([[0, 7, 300] for _ in range(B * Hq)])
    sp, si = _csr([list(range(20)) + [77, 400] for _ in range(B * Hq)])
    a = _run(q, k, v, bp, bi, cp, ci, sp, si)
    b = _run(q, k, v, bp, bi, cp, ci, sp, si)
    assert all(bool((x == y).all()) for x, y in zip(a, b))


def test_vslash_128k_sampled_rows():
    """The 128K vertical-slash workload (B 1, Hq 32, Hkv 8, D 128), in the launch the bench
    times: every head's output on 1024 sampled rows (the first 64, the last 64 and 896 drawn)
    against the oracle, each row scored over the keys its columns and slash lines reach (the
    oracle's masks), which is exactly the set the mask leaves visible."""
    import torch
    w = WORKLOADS["vslash_128k"]
    say(f"vslash full size {w.name}")
    q, k, v = make_qkv(w)
    sp, si, cp, ci = make_vslash_lists(w.B, w.Hq, w.Lk, 1000 * w.index + 3)
    bp, bi = _no_blocks(w.B, w.Hq, w.Lq)
    o, lse = _run(q, k, v, bp, bi, cp, ci, sp, si, scale=w.scale)
    rows = sampled_rows(w.Lq, 1024, 1000 * w.index + 4)
    g = w.Hq // w.Hkv
    no_blocks = lambda qb: np.zeros(0, np.int64)
    for h in range(w.Hq):
        allowed = (A.blocksparse_row_mask(rows, w.Lk, no_blocks, ci[cp[h]:cp[h + 1]])
                   | A.slash_row_mask(rows, w.Lq, w.Lk, si[sp[h]:sp[h + 1]]))
        kh = k[0, :, h // g].double().numpy()
        vh = v[0, :, h // g].double().numpy()
        qh = q[0, rows, h].double().numpy()
        ro, rl = [], []
        for i, r in enumerate(rows):
            orow, lrow = A.attention_rows_over_keys(qh[[i]], [r], kh, vh,
                                                    A.effective_scale(w.scale),
                                                    np.nonzero(allowed[i])[0], w.Lq, w.Lk, True)
            ro.append(orow)
            rl.append(lrow)
        del allowed
        check_parity(o[0, rows, h].float().cpu().double().numpy(), np.concatenate(ro),
                     lse[0, h, rows].cpu().double().numpy(), np.concatenate(rl),
                     f"vslash_128k h={h}")


def test_vslash_reference_jumps():
    """Rising / falling / alternating scores (as in the block-sparse reference-jump test) over
    columns and slash lines only: the first keys a row meets come from phase 2 or phase 3, and
    later lines raise the row's maximum by far more than fp32 weights can hold."""
    import torch
    say("vslash reference jumps")
    B, Hq, Hkv, L, D = 1, 6, 3, 640, 128
    u = torch.full((D,), 1.0)
    t = 20.0 * (torch.arange(L) // 32).float()
    q = (u.expand(B, L, Hq, D) + 0.1 * randn_bf16((B, L, Hq, D), 9900).float()).to(torch.bfloat16)
    kf = 0.1 * randn_bf16((B, L, Hkv, D), 9901).float()
    kf[:, :, 0] += t[:, None] / 8.0
    kf[:, :, 1] += t.flip(0)[:, None] / 8.0
    kf[:, :, 2] += (t[:, None] / 8.0) * ((torch.arange(L) % 64) < 32).float()[:, None]
    k = kf.to(torch.bfloat16)
    v = randn_bf16((B, L, Hkv, D), 9902) * 0.5  # peaked rows: keeps |O| < 4
    rng = np.random.default_rng(9903)
    bp, bi = _no_blocks(B, Hq, L)
    cp, ci = _csr([rng.choice(L, 40, replace=False) for _ in range(B * Hq)])
    sp, si = _csr([np.concatenate([np.arange(0, 8), rng.integers(8, L, 20)])
                   for _ in range(B * Hq)])
    _compare(q, k, v, bp, bi, cp, ci, sp, si, "vslash jumps")

"""GPU parity at GQA ratios beyond the sweeps' 1..8: 16, 32 and 64 query heads per KV head
(multi-query attention at the far end), and decode shapes with more than 16 query columns per
KV head (heads of the group times query tokens). Decode then runs one workgroup over two
16-column blocks, up to four such workgroups per KV head (g * Lq up to 128 columns), and
prefill and block-sparse map many query heads onto one K/V stream. Compared element by element
with the fp64 oracle."""

import numpy as np
import pytest

from oracle import attention as A
from tests.helpers import check_parity, say, to_f64
from workloads import randn_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _qkv(B, Lq, Lk, Hq, Hkv, D, seed):
    return (randn_bf16((B, Lq, Hq, D), seed), randn_bf16((B, Lk, Hkv, D), seed + 1),
            randn_bf16((B, Lk, Hkv, D), seed + 2))


@pytest.mark.parametrize("shape", [(1, 16, 1, 333, 128), (2, 32, 1, 200, 64), (1, 64, 2, 130, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_prefill_wide_groups(shape):
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, L, D = shape
    say(f"prefill, {Hq // Hkv} query heads per KV head: {shape}")
    q, k, v = _qkv(B, L, L, Hq, Hkv, D, 9990 + Hq)
    o = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    S.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), o, lse, causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5),
                               True)
    check_parity(to_f64(o), o_ref, to_f64(lse), l_ref, f"prefill wide {shape}")


@pytest.mark.parametrize("shape", [(4, 16, 1, 1, 3000, 128), (2, 32, 1, 2, 1500, 128),
                                   (3, 64, 1, 2, 777, 64), (2, 64, 2, 1, 4100, 128),
                                   # 17..32 columns per KV head: one workgroup takes both
                                   # 16-column blocks, the second one partly filled
                                   (3, 24, 2, 2, 999, 128), (2, 8, 1, 3, 2000, 128),
                                   (1, 32, 4, 4, 513, 64), (2, 40, 2, 1, 1000, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_decode_wide_groups(shape):
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, Lq, Lk, D = shape
    say(f"decode, {Hq // Hkv} query heads per KV head: {shape}, "
        f"{S.attn_splitkv_num_splits(B, Hq, Hkv, Lq, Lk, D, D)} splits")
    q, k, v = _qkv(B, Lq, Lk, Hq, Hkv, D, 9995 + Hq + Lq)
    o = torch.empty((B, Lq, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    S.attn_fwd_decode(q.to(DEV), k.to(DEV), v.to(DEV), o, lse, causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5),
                               True)
    check_parity(to_f64(o), o_ref, to_f64(lse), l_ref, f"decode wide {shape}")


def test_blocksparse_wide_groups():
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, L, D = 1, 32, 1, 700, 128
    say(f"block-sparse, 32 query heads per KV head, L {L}")
    q, k, v = _qkv(B, L, L, Hq, Hkv, D, 9999)
    rng = np.random.default_rng(9999)
    nqb = -(-L // 64)
    ptr, idx = [0], []
    for _ in range(B * Hq):
        for qb in range(nqb):
            blks = sorted({0, qb} | {int(x) for x in rng.integers(0, qb + 1, 2)})
            idx.extend(blks)
            ptr.append(ptr[-1] + len(blks))
    cptr, cidx = [0], []
    for _ in range(B * Hq):
        c = np.unique(rng.integers(0, L, 24))
        cidx.extend(int(x) for x in c)
        cptr.append(cptr[-1] + c.size)
    bp, bi = np.asarray(ptr, np.int32), np.asarray(idx, np.int32)
    cp, ci = np.asarray(cptr, np.int32), np.asarray(cidx, np.int32)
    S.attn_blocksparse_check(bp, bi, cp, ci, B, Hq, L, L)
    dev = lambda x: torch.as_tensor(x).to(DEV)
    o = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    S.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), o, dev(bp), dev(bi), dev(cp),
                           dev(ci), lse=lse, causal=True)
    torch.cuda.synchronize()
    fn = A.csr_allowed_fn(bp, bi, cp, ci, hq=Hq, nqb=nqb, lk=L)
    o_ref, l_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5),
                               True, allowed_fn=fn)
    check_parity(to_f64(o), o_ref, to_f64(lse), l_ref, "block-sparse wide groups")

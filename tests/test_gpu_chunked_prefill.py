"""GPU parity of split-KV over prefill-shaped query blocks (D = 64 or 128; at least 128 query
rows, or 64 over at least 8192 keys), which the library computes with the dense prefill
kernel's split form: a short query chunk against a longer cache (chunked prefill, bottom-right
causal), through attn_fwd_splitkv (the per-split partials, compared with the oracle's
partials) and through the one-call attn_fwd_decode (split partials plus the LSE combine, or one
split written directly)."""

import numpy as np
import pytest

from oracle import attention as A
from tests.helpers import check_parity, say, to_f64
from workloads import randn_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _qkv(B, Hq, Hkv, Lq, Lk, D, seed):
    return (randn_bf16((B, Lq, Hq, D), seed), randn_bf16((B, Lk, Hkv, D), seed + 1),
            randn_bf16((B, Lk, Hkv, D), seed + 2))


@pytest.mark.parametrize("shape", [
    # B, Hq, Hkv, Lq, Lk, D, causal, splits
    (1, 8, 2, 300, 5000, 128, True, 4),     # ragged rows and keys, the diagonal in the last split
    (2, 4, 1, 256, 3000, 64, False, 3),
    (1, 4, 4, 129, 700, 128, True, 11),     # 64-key splits, the last one of 60 keys
    (1, 4, 2, 200, 256, 128, True, 3),      # 128-key splits: the third is empty
    (1, 8, 2, 400, 300, 128, True, 2),      # Lq > Lk: the first rows see no key at all
    (1, 4, 1, 64, 8192, 64, False, 5),      # 64 rows over 8K keys: a half-filled row tile
], ids=lambda s: "x".join(map(str, s)))
def test_dense_split_partials_match_oracle(shape):
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, Lq, Lk, D, causal, splits = shape
    say(f"dense split partials {shape}")
    q, k, v = _qkv(B, Hq, Hkv, Lq, Lk, D, 9600 + Lq)
    op = torch.full((splits, B, Hq, Lq, D), float("nan"), dtype=torch.float32, device=DEV)
    lp = torch.full((splits, B, Hq, Lq), float("nan"), dtype=torch.float32, device=DEV)
    S.attn_fwd_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), op, lp, causal=causal, scale=D ** -0.5)
    torch.cuda.synchronize()
    op_ref, lp_ref = A.splitkv_partials(to_f64(q), to_f64(k), to_f64(v),
                                        A.effective_scale(D ** -0.5), causal, splits)
    check_parity(to_f64(op), op_ref, to_f64(lp), lp_ref, f"dense split partials {shape}")


@pytest.mark.parametrize("shape", [
    # B, Hq, Hkv, Lq, Lk, D, causal
    (1, 16, 4, 384, 3000, 128, True),       # a chunk against a longer cache: several splits
    (2, 8, 2, 200, 3000, 64, True),
    (1, 16, 4, 1000, 1000, 128, True),      # square: one split, the prefill kernel directly
    (1, 8, 8, 150, 2500, 128, False),
    (1, 8, 2, 100, 9000, 128, True),        # under 128 rows, over 8K keys: the split form too
], ids=lambda s: "x".join(map(str, s)))
def test_chunked_prefill_one_call(shape):
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, Lq, Lk, D, causal = shape
    nsp = S.attn_splitkv_num_splits(B, Hq, Hkv, Lq, Lk, D, D)
    say(f"chunked prefill {shape}: {nsp} splits")
    q, k, v = _qkv(B, Hq, Hkv, Lq, Lk, D, 9700 + Lq)
    o = torch.empty((B, Lq, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    S.attn_fwd_decode(q.to(DEV), k.to(DEV), v.to(DEV), o, lse, causal=causal, scale=D ** -0.5)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5),
                                 causal)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"chunked prefill {shape}")


def test_chunked_prefill_equals_prefill_kernel_when_one_split():
    """With one split the one-call path runs the prefill kernel itself: bit-equal to attn_fwd."""
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, Lq, Lk, D = 1, 16, 4, 1000, 1000, 128
    assert S.attn_splitkv_num_splits(B, Hq, Hkv, Lq, Lk, D, D) == 1
    say("chunked prefill, one split, against attn_fwd")
    q, k, v = [t.to(DEV) for t in _qkv(B, Hq, Hkv, Lq, Lk, D, 9800)]
    o1 = torch.empty((B, Lq, Hq, D), dtype=torch.bfloat16, device=DEV)
    l1 = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    S.attn_fwd_decode(q, k, v, o1, l1, causal=True)
    S.attn_fwd(q, k, v, o2, l2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)

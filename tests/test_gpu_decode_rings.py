"""GPU parity of both D = 128 split-KV decode rings against the fp64 oracle, through
attn_fwd_splitkv + attn_combine_lse with the split count forced: grids of at most one workgroup
per CU run the 4-stage ring of 32-key tiles, larger grids the 2-stage ring of 64-key tiles.
Cache lengths are ragged (a 32-key tile or a 64-key tile cut short, splits whose last tile is a
single key, lengths below one tile), with one to three query tokens under the bottom-right
causal mask."""

import pytest

from oracle import attention as A
from tests.helpers import check_parity, say, to_f64
from workloads import randn_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    # B, Hq, Hkv, Lq, Lk, splits, causal; workgroups = B * Hkv * splits (one 16-column block)
    (4, 32, 8, 1, 4096 + 37, 8, False),     # 256: the 32-key ring, a ragged last split
    (4, 32, 8, 1, 4096 + 37, 16, False),    # 512: the 64-key ring, same keys
    (40, 8, 2, 3, 1000, 3, True),           # 240: 32-key ring, last split 232 keys
    (40, 8, 2, 3, 1000, 4, True),           # 320: 64-key ring, last split 232 keys
    (1, 16, 4, 2, 33, 1, True),             # one split under one 32-key tile
    (3, 16, 4, 1, 64 * 21 + 1, 21, False),  # 252: 128-key splits, the 11th holds 65 keys, ten empty
    (16, 32, 8, 1, 4096, 2, False),         # the batched GQA decode workload's grid (256)
    (16, 32, 8, 1, 4096, 4, False),         # 512 workgroups: 64-key ring
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_d128_decode_rings(case):
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, Lq, Lk, splits, causal = case
    D = 128
    say(f"D128 decode ring case {case}: {B * Hkv * splits} workgroups")
    q = randn_bf16((B, Lq, Hq, D), 9900 + Lk)
    k = randn_bf16((B, Lk, Hkv, D), 9901 + Lk)
    v = randn_bf16((B, Lk, Hkv, D), 9902 + Lk)
    o = torch.empty((B, Lq, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    S.splitkv_decode(q.to(DEV), k.to(DEV), v.to(DEV), o, lse, causal=causal, scale=D ** -0.5,
                     num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5),
                                 causal)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"D128 ring {case}")

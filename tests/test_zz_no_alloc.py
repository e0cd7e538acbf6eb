"""GPU check of attn_fwd_decode_noalloc (the allocation-free decode entry point) through the C
ABI: its O and LSE equal attn_fwd_decode's bit for bit (same kernels and split count; the
partials only live in the library's scratch array instead of a caller workspace), and both meet
the oracle's parity bar. Two calls in a row, the second with a smaller input, so the second
reads partials over the first call's leftovers in the shared scratch."""

import numpy as np
import pytest

from oracle import attention as A
from tests.helpers import check_parity, say, to_f64
from workloads import randn_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    # B, Hq, Hkv, Lq, Lk, Dqk, Dv, causal
    (16, 32, 8, 1, 4096, 128, 128, False),   # the batched GQA decode workload's shape
    (3, 8, 2, 2, 1500, 128, 128, True),      # smaller, two query tokens, bottom-right causal
]
MLA_CASES = [
    (8, 16, 1, 1, 65536, 576, 512, False),   # the MLA decode workload's shape (32 splits)
    (2, 16, 1, 2, 3000, 576, 512, True),     # smaller
]


def _pair(shape, seed):
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, Lq, Lk, Dqk, Dv, causal = shape
    q = randn_bf16((B, Lq, Hq, Dqk), seed)
    k = randn_bf16((B, Lk, Hkv, Dqk), seed + 1)
    mla = Dqk != Dv
    v = None if mla else randn_bf16((B, Lk, Hkv, Dv), seed + 2)
    qd, kd = q.to(DEV), k.to(DEV)
    vd = kd[..., :Dv] if mla else v.to(DEV)
    scale = (192 if mla else Dqk) ** -0.5
    if S.attn_splitkv_num_splits(B, Hq, Hkv, Lq, Lk, Dqk, Dv) > 1:
        assert S.attn_decode_workspace_bytes(B, Hq, Hkv, Lq, Lk, Dqk, Dv) <= \
            S.ATTN_DECODE_SCRATCH_BYTES
    o_ref = torch.empty((B, Lq, Hq, Dv), dtype=torch.bfloat16, device=DEV)
    l_ref = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    S.attn_fwd_decode(qd, kd, vd, o_ref, l_ref, causal=causal, scale=scale)
    o = torch.full((B, Lq, Hq, Dv), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device=DEV)
    S.attn_fwd_decode_noalloc(qd, kd, vd, o, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), f"{shape}: O differs from attn_fwd_decode's"
    assert torch.equal(lse, l_ref), f"{shape}: LSE differs from attn_fwd_decode's"
    vf = A.mla_value_view(to_f64(k), Dv) if mla else to_f64(v)
    o64, l64 = A.attention(to_f64(q), to_f64(k), vf, A.effective_scale(scale), causal)
    check_parity(to_f64(o), o64, to_f64(lse), l64, f"noalloc {shape}")


@pytest.mark.parametrize("cases", [CASES, MLA_CASES], ids=["gqa", "mla"])
def test_noalloc_decode_equals_workspace_decode(cases):
    for i, shape in enumerate(cases):        # second call smaller than the first
        say(f"noalloc decode {shape}")
        _pair(shape, 9700 + 10 * i)


def test_noalloc_rejects_sizes_beyond_scratch():
    """MLA decode with 64 heads, 16 query tokens and 2048 keys needs 8 splits and more
    partials than the scratch holds: WORKSPACE, and nothing written."""
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, Lq, Lk, D = 1, 64, 1, 16, 2048, 576
    assert S.attn_splitkv_num_splits(B, Hq, Hkv, Lq, Lk, D, 512) > 1
    assert S.attn_decode_workspace_bytes(B, Hq, Hkv, Lq, Lk, D, 512) > S.ATTN_DECODE_SCRATCH_BYTES
    say("noalloc decode beyond the scratch size")
    q = torch.zeros((B, Lq, Hq, D), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((B, Lk, Hkv, D), dtype=torch.bfloat16, device=DEV)
    o = torch.zeros((B, Lq, Hq, 512), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(S.AttnError) as e:
        S.attn_fwd_decode_noalloc(q, k, k[..., :512], o)
    assert e.value.status == S.ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert float(o.abs().max()) == 0.0, "nothing may be written on an error"


def test_noalloc_one_split_beyond_scratch_size():
    """One split (1024 (b, KV head) units fill the GPU): O and LSE are written directly, no
    partials exist, so a size whose workspace would exceed the scratch is accepted."""
    B, Hq, Hkv, Lq, Lk, D = 1024, 32, 1, 4, 256, 128
    import sparse_attention_attn_amd as S
    assert S.attn_splitkv_num_splits(B, Hq, Hkv, Lq, Lk, D, D) == 1
    assert S.attn_decode_workspace_bytes(B, Hq, Hkv, Lq, Lk, D, D) > S.ATTN_DECODE_SCRATCH_BYTES
    say("noalloc decode, one split, large batch")
    _pair((B, Hq, Hkv, Lq, Lk, D, D, True), 9800)

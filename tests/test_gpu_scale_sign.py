"""GPU parity for negative and zero softmax scales (dense prefill, split-KV decode including the
MLA shape, block-sparse and vertical-slash), against the fp64 oracle, through the C ABI.

softmax(scale·QKᵀ + mask) is defined for every finite scale. A negative scale reverses the order
of the scores (the row maximum of scale·s comes from the smallest s), and masked keys must still
get weight 0; scale 0 gives every visible key the same weight, so O is the mean of the visible
value rows and LSE = ln(number of visible keys).
"""

import numpy as np
import pytest

from oracle import attention as A
from tests.helpers import check_parity, say, to_f64
from workloads import make_blocksparse_lists, randn_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALES = [-0.125, -1.0, 0.0]


def _qkv(B, Lq, Lk, Hq, Hkv, Dqk, Dv, seed):
    # V halved (exact in bf16): a large |scale| makes rows peaked, O then follows single value
    # rows, and |O| stays below 4, where bf16 output rounding alone could exceed 1e-2.
    return (randn_bf16((B, Lq, Hq, Dqk), seed), randn_bf16((B, Lk, Hkv, Dqk), seed + 1),
            randn_bf16((B, Lk, Hkv, Dv), seed + 2) * 0.5)


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("shape", [(1, 4, 2, 200, 200, 128, True), (2, 8, 2, 130, 333, 64, True),
                                   (1, 2, 1, 97, 300, 128, False)],
                         ids=lambda s: "x".join(map(str, s)))
def test_prefill_scale_sign(shape, scale):
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, Lq, Lk, D, causal = shape
    say(f"prefill scale {scale} {shape}")
    q, k, v = _qkv(B, Lq, Lk, Hq, Hkv, D, D, 9400 + sum(shape))
    o = torch.empty((B, Lq, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    S.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), o, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(scale), causal)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"prefill scale {scale}")


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("mla", [False, True], ids=["gqa", "mla"])
def test_decode_scale_sign(mla, scale):
    import torch
    import sparse_attention_attn_amd as S
    say(f"decode scale {scale} mla={mla}")
    if mla:
        B, Hq, Hkv, Lq, Lk, Dqk, Dv = 2, 16, 1, 2, 1500, 576, 512
    else:
        B, Hq, Hkv, Lq, Lk, Dqk, Dv = 3, 8, 2, 1, 1000, 128, 128
    q, k, v = _qkv(B, Lq, Lk, Hq, Hkv, Dqk, Dv, 9500 + int(mla))
    if mla:
        k = k * 0.5  # V is K's first 512 columns: halved like V above
    kd = k.to(DEV)
    vd = kd[..., :512] if mla else v.to(DEV)
    vf = A.mla_value_view(to_f64(k), 512) if mla else to_f64(v)
    o = torch.empty((B, Lq, Hq, Dv), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    S.splitkv_decode(q.to(DEV), kd, vd, o, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), vf, A.effective_scale(scale), True)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"decode scale {scale}")


def _dev(x):
    import torch
    return torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32)).to(DEV)


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("slash", [False, True], ids=["blocksparse", "vslash"])
def test_sparse_scale_sign(slash, scale):
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, L, D = 1, 4, 2, 1000, 128
    say(f"sparse scale {scale} slash={slash}")
    q, k, v = _qkv(B, L, L, Hq, Hkv, D, D, 9600 + int(slash))
    bp, bi, cp, ci = make_blocksparse_lists(B, Hq, L, L, 9610, local_blocks=3, p_extra=0.1,
                                           n_cols=60)
    o = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    if slash:
        rng = np.random.default_rng(9620)
        per_head = [np.unique(np.concatenate([np.arange(0, 40), rng.integers(40, L, 10)]))
                    for _ in range(B * Hq)]
        sp = np.asarray([0] + list(np.cumsum([len(x) for x in per_head])), np.int32)
        si = np.concatenate(per_head).astype(np.int32)
        S.attn_fwd_vertical_slash(q.to(DEV), k.to(DEV), v.to(DEV), o, _dev(bp), _dev(bi),
                                  _dev(cp), _dev(ci), _dev(sp), _dev(si), lse=lse, causal=True,
                                  scale=scale)
        fn = A.vslash_allowed_fn(bp, bi, cp, ci, sp, si, Hq, -(-L // 64), L, L)
    else:
        S.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), o, _dev(bp), _dev(bi), _dev(cp),
                               _dev(ci), lse=lse, causal=True, scale=scale)
        fn = A.csr_allowed_fn(bp, bi, cp, ci, hq=Hq, nqb=-(-L // 64), lk=L)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(scale), True,
                                 allowed_fn=fn)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"sparse scale {scale}")

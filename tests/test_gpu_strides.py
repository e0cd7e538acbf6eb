"""GPU parity with non-contiguous layouts, through the stride arguments of the C ABI: a
head-major KV cache ([B, Hkv, Lk, D] viewed as [B, Lk, Hkv, D]) for split-KV decode, an MLA
latent cache with padded rows, packed Q/K/V buffers for block-sparse, vertical-slash and the
index builders, and O written into a wider buffer whose other columns must stay untouched."""

import numpy as np
import pytest

from oracle import attention as A
from tests.helpers import check_parity, say, to_f64
from workloads import make_blocksparse_lists, randn_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dev(x):
    import torch
    return torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32)).to(DEV)


def _wide_out(B, L, Hq, Dv):
    import torch
    obuf = torch.zeros((B, L, Hq + 3, Dv), dtype=torch.bfloat16, device=DEV)
    return obuf, obuf[:, :, 1:1 + Hq]


def _untouched(obuf, Hq):
    assert float(obuf[:, :, 0].abs().max()) == 0.0
    assert float(obuf[:, :, 1 + Hq:].abs().max()) == 0.0


def test_decode_head_major_cache():
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, Lq, Lk, D = 3, 8, 2, 2, 900, 128
    say("decode head-major cache")
    q = randn_bf16((B, Lq, Hq, D), 9950)
    kc = randn_bf16((B, Hkv, Lk, D), 9951)  # cache stored head-major
    vc = randn_bf16((B, Hkv, Lk, D), 9952)
    kd = kc.to(DEV).permute(0, 2, 1, 3)  # [B, Lk, Hkv, D] view: stride_l = D, stride_h = Lk*D
    vd = vc.to(DEV).permute(0, 2, 1, 3)
    obuf, od = _wide_out(B, Lq, Hq, D)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    S.splitkv_decode(q.to(DEV), kd, vd, od, lse, causal=True, scale=D ** -0.5)
    torch.cuda.synchronize()
    k = kc.permute(0, 2, 1, 3).contiguous()
    v = vc.permute(0, 2, 1, 3).contiguous()
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5), True)
    check_parity(to_f64(od), o_ref, to_f64(lse), lse_ref, "decode head-major")
    _untouched(obuf, Hq)


def test_decode_mla_padded_rows():
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Lq, Lk = 2, 16, 1, 1300
    say("decode MLA latent cache with padded rows")
    q = randn_bf16((B, Lq, Hq, 576), 9960)
    cache = randn_bf16((B, Lk, 1, 640), 9961)  # rows padded to 640 elements
    kd = cache.to(DEV)[..., :576]
    obuf, od = _wide_out(B, Lq, Hq, 512)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    S.splitkv_decode(q.to(DEV), kd, kd[..., :512], od, lse, causal=True, scale=192 ** -0.5)
    torch.cuda.synchronize()
    kf = to_f64(cache[..., :576].contiguous())
    o_ref, lse_ref = A.attention(to_f64(q), kf, A.mla_value_view(kf, 512),
                                 A.effective_scale(192 ** -0.5), True)
    check_parity(to_f64(od), o_ref, to_f64(lse), lse_ref, "decode MLA padded")
    _untouched(obuf, Hq)


def _packed(B, L, Hq, Hkv, D, seed):
    packed = randn_bf16((B, L, Hq + 2 * Hkv, D), seed)
    pd = packed.to(DEV)
    host = (packed[:, :, :Hq].contiguous(), packed[:, :, Hq:Hq + Hkv].contiguous(),
            packed[:, :, Hq + Hkv:].contiguous())
    dev = (pd[:, :, :Hq], pd[:, :, Hq:Hq + Hkv], pd[:, :, Hq + Hkv:])
    return host, dev


@pytest.mark.parametrize("slash", [False, True], ids=["blocksparse", "vslash"])
def test_sparse_packed_qkv(slash):
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, L, D = 2, 4, 2, 700, 128
    say(f"sparse packed qkv slash={slash}")
    (q, k, v), (qd, kd, vd) = _packed(B, L, Hq, Hkv, D, 9970 + int(slash))
    bp, bi, cp, ci = make_blocksparse_lists(B, Hq, L, L, 9975, local_blocks=3, p_extra=0.15,
                                           n_cols=50)
    obuf, od = _wide_out(B, L, Hq, D)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    if slash:
        rng = np.random.default_rng(9976)
        offs = [np.unique(np.concatenate([np.arange(0, 20), rng.integers(20, L, 12)]))
                for _ in range(B * Hq)]
        sp = np.asarray([0] + list(np.cumsum([x.size for x in offs])), np.int32)
        si = np.concatenate(offs).astype(np.int32)
        S.attn_fwd_vertical_slash(qd, kd, vd, od, _dev(bp), _dev(bi), _dev(cp), _dev(ci),
                                  _dev(sp), _dev(si), lse=lse, causal=True, scale=D ** -0.5)
        fn = A.vslash_allowed_fn(bp, bi, cp, ci, sp, si, Hq, -(-L // 64), L, L)
    else:
        S.attn_fwd_blocksparse(qd, kd, vd, od, _dev(bp), _dev(bi), _dev(cp), _dev(ci), lse=lse,
                               causal=True, scale=D ** -0.5)
        fn = A.csr_allowed_fn(bp, bi, cp, ci, hq=Hq, nqb=-(-L // 64), lk=L)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5),
                                 True, allowed_fn=fn)
    check_parity(to_f64(od), o_ref, to_f64(lse), lse_ref, f"sparse packed slash={slash}")
    _untouched(obuf, Hq)


def test_index_builder_packed_inputs_match_contiguous():
    """The block/column index built from packed (strided) Q and K equals the one built from
    contiguous copies of the same tensors (the builder's arithmetic is checked against the
    oracle in test_gpu_sparse_index; here only the stride handling differs)."""
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, L, D = 1, 4, 2, 1000, 128
    say("index builder packed inputs")
    (q, k, _), (qd, kd, _) = _packed(B, L, Hq, Hkv, D, 9980)
    a = S.attn_build_sparse_index(qd, kd, 6, 40)
    b = S.attn_build_sparse_index(q.to(DEV), k.to(DEV), 6, 40)
    for x, y in zip(a, b):
        assert x.shape == y.shape and bool((x == y).all())
    c = S.attn_build_vslash_index(qd, kd, 30, 20)
    d = S.attn_build_vslash_index(q.to(DEV), k.to(DEV), 30, 20)
    for x, y in zip(c, d):
        assert x.shape == y.shape and bool((x == y).all())

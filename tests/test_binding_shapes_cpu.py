"""CPU checks of the Python binding's shape, size and device checks: a tensor whose shape
disagrees with the sizes a wrapper passes to the C ABI is rejected with ValueError before any
pointer is taken (the C side sees raw pointers and cannot check buffer sizes). These run on CPU
tensors, which the binding would refuse later anyway, so every case here is caught by the
shape checks themselves."""

import pytest
import torch

import sparse_attention_attn_amd as S

bf = torch.bfloat16
f32 = torch.float32
i32 = torch.int32


def _qkvo(B=2, Lq=8, Lk=16, Hq=4, Hkv=2, D=128, Dv=None):
    Dv = Dv or D
    return (torch.zeros(B, Lq, Hq, D, dtype=bf), torch.zeros(B, Lk, Hkv, D, dtype=bf),
            torch.zeros(B, Lk, Hkv, Dv, dtype=bf), torch.zeros(B, Lq, Hq, Dv, dtype=bf))


def _raises(fn, frag):
    with pytest.raises(ValueError, match=frag):
        fn()


def test_attn_fwd_shape_checks():
    q, k, v, o = _qkvo()
    _raises(lambda: S.attn_fwd(q, k, v, torch.zeros(2, 8, 4, 64, dtype=bf)), "o must have shape")
    _raises(lambda: S.attn_fwd(q, k, v[:1], o), "batch sizes differ")
    _raises(lambda: S.attn_fwd(q, k, v[:, :15], o), "must agree")
    _raises(lambda: S.attn_fwd(q, k[..., :64], v, o), "head dim")
    _raises(lambda: S.attn_fwd(q, k, v, o, torch.zeros(2 * 4 * 8 - 1, dtype=f32)), "lse must hold")
    _raises(lambda: S.attn_fwd(q[0], k, v, o), r"\[B, L, H, D\]")


def test_splitkv_and_combine_shape_checks():
    q, k, v, o = _qkvo(Lq=1)
    op = torch.zeros(3, 2, 4, 1, 128, dtype=f32)
    lp = torch.zeros(3, 2, 4, 1, dtype=f32)
    _raises(lambda: S.attn_fwd_splitkv(q, k, v, op[:, :1], lp), "o_part must have shape")
    _raises(lambda: S.attn_fwd_splitkv(q, k, v, op, lp[:2]), "lse_part must have shape")
    _raises(lambda: S.attn_combine_lse(op, lp[:, :, :3], o), "lse_part must have shape")
    _raises(lambda: S.attn_combine_lse(op, lp, o[:, :, :2]), "o must have shape")
    _raises(lambda: S.attn_combine_lse(op, lp, o, torch.zeros(9, dtype=f32)), "lse must hold")


def test_decode_shape_and_workspace_checks():
    q, k, v, o = _qkvo(Lq=1, Lk=4096)
    need = S.attn_decode_workspace_bytes(2, 4, 2, 1, 4096, 128, 128)
    ws = torch.zeros(need - 256, dtype=torch.uint8)
    _raises(lambda: S.attn_fwd_decode(q, k, v, o, workspace=ws), "workspace must hold")
    _raises(lambda: S.attn_fwd_decode(q, k, v, o[:1], workspace=ws), "o must have shape")


def test_blocksparse_list_size_checks():
    q, k, v, o = _qkvo(Lq=200, Lk=200)
    nqb = 4
    bp = torch.zeros(2 * 4 * nqb + 1, dtype=i32)
    bi = torch.zeros(1, dtype=i32)
    cp = torch.zeros(2 * 4 + 1, dtype=i32)
    ci = torch.zeros(1, dtype=i32)
    _raises(lambda: S.attn_fwd_blocksparse(q, k, v, o, bp[:-1], bi, cp, ci), "blk_ptr must hold")
    _raises(lambda: S.attn_fwd_blocksparse(q, k, v, o, bp, bi, cp[:-1], ci), "col_ptr must hold")
    sp = torch.zeros(2 * 4 + 1, dtype=i32)
    _raises(lambda: S.attn_fwd_vertical_slash(q, k, v, o, bp, bi, cp, ci, sp[:-1], ci),
            "slash_ptr must hold")
    ws = torch.zeros(8, dtype=torch.uint8)
    _raises(lambda: S.attn_fwd_vertical_slash(q, k, v, o, bp, bi, cp, ci, sp, ci, workspace=ws),
            "workspace must hold")


def test_index_builder_size_checks():
    B, L, Hq, Hkv, D = 1, 300, 4, 2, 128
    q = torch.zeros(B, L, Hq, D, dtype=bf)
    k = torch.zeros(B, L, Hkv, D, dtype=bf)
    _raises(lambda: S.attn_build_sparse_index(q, k[:, :299], 4, 10), "must be \\[B, L, Hkv, D\\]")
    nb, nc = S.attn_sparse_index_sizes(B, Hq, L, 4, 10)
    outs = (torch.zeros(B * Hq * 5 + 1, dtype=i32), torch.zeros(nb - 1, dtype=i32),
            torch.zeros(B * Hq + 1, dtype=i32), torch.zeros(nc, dtype=i32))
    _raises(lambda: S.attn_build_sparse_index(q, k, 4, 10, outputs=outs), "blk_idx must hold")
    outs_vs = (torch.zeros(B * Hq + 1, dtype=i32), torch.zeros(B * Hq * 10, dtype=i32),
               torch.zeros(B * Hq + 1, dtype=i32), torch.zeros(B * Hq * 7 - 1, dtype=i32))
    _raises(lambda: S.attn_build_vslash_index(q, k, 10, 7, outputs=outs_vs), "slash_idx must hold")
    ws = torch.zeros(16, dtype=torch.uint8)
    _raises(lambda: S.attn_build_vslash_index(q, k, 10, 7, outputs=outs_vs[:3] +
                                              (torch.zeros(B * Hq * 7, dtype=i32),), workspace=ws),
            "workspace must hold")

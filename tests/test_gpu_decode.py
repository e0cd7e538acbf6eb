"""GPU parity of the split-KV decode path (attn_fwd_splitkv + attn_combine_lse) and of the
combine alone, against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest

from oracle import attention as A
from tests.helpers import check_parity, say, to_f64
from workloads import ETAP_GRID, WORKLOADS, make_qkv, randn_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _decode(q, k, v, causal, scale, num_splits=None):
    import torch
    import sparse_attention_attn_amd as S
    B, Lq, Hq, _ = q.shape
    Dv = v.shape[3]
    o = torch.empty((B, Lq, Hq, Dv), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    S.splitkv_decode(q, k, v, o, lse, causal=causal, scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return o, lse


def test_gqa_decode_workload_full():
    w = WORKLOADS["gqa_decode_4k"]
    say(f"gqa_decode_4k full {w}")
    q, k, v = make_qkv(w)
    o, lse = _decode(q.to(DEV), k.to(DEV), v.to(DEV), False, w.scale)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(w.scale), False)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, "gqa_decode_4k")


def test_mla_decode_workload_full():
    """MLA latent shape: V is the first 512 columns of K (a view, same memory)."""
    w = WORKLOADS["mla_decode_64k"]
    say(f"mla_decode_64k full {w}")
    q, k, _ = make_qkv(w)
    kd = k.to(DEV)
    o, lse = _decode(q.to(DEV), kd, kd[..., :512], False, w.scale)
    kf = to_f64(k)
    o_ref, lse_ref = A.attention(to_f64(q), kf, A.mla_value_view(kf, 512),
                                 A.effective_scale(w.scale), False)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, "mla_decode_64k")


@pytest.mark.parametrize("splits", [1, 2, 7, 64])
def test_split_invariance_gqa(splits):
    """Any split count gives the oracle's result (and the split-count-independent LSE)."""
    B, Hq, Hkv, Lk, D = 3, 8, 2, 4096 + 37, 128
    say(f"split invariance S={splits} B={B} Hq={Hq} Hkv={Hkv} Lk={Lk}")
    q = randn_bf16((B, 1, Hq, D), 8000)
    k = randn_bf16((B, Lk, Hkv, D), 8001)
    v = randn_bf16((B, Lk, Hkv, D), 8002)
    o, lse = _decode(q.to(DEV), k.to(DEV), v.to(DEV), False, D ** -0.5, num_splits=splits)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5), False)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"splits={splits}")


def test_splitkv_partials_match_oracle_partials():
    """The per-split partials themselves (O_s, LSE_s), including empty trailing splits."""
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, Lq, Lk, D = 2, 4, 1, 1, 256, 64
    splits = 3   # chunk 128 -> third split is empty
    say(f"partials S={splits}")
    q = randn_bf16((B, Lq, Hq, D), 8100)
    k = randn_bf16((B, Lk, Hkv, D), 8101)
    v = randn_bf16((B, Lk, Hkv, D), 8102)
    op = torch.empty((splits, B, Hq, Lq, D), dtype=torch.float32, device=DEV)
    lp = torch.empty((splits, B, Hq, Lq), dtype=torch.float32, device=DEV)
    S.attn_fwd_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), op, lp, causal=False, scale=0.125)
    torch.cuda.synchronize()
    op_ref, lp_ref = A.splitkv_partials(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(0.125),
                                        False, splits)
    check_parity(to_f64(op), op_ref, to_f64(lp), lp_ref, "partials")
    assert bool(torch.isneginf(lp[2]).all()) and float(op[2].abs().max()) == 0.0


@pytest.mark.parametrize("shape", [
    # B, Hq, Hkv, Lq, Lk, D, causal, splits
    (3, 16, 8, 2, 2389, 128, True, 5),    # 8 KV heads: the walk starts mid-split; the ragged
                                          # last tile (341 keys in the last split) and the
                                          # causal edge come first or in the middle
    (2, 8, 2, 3, 1000, 64, True, 4),      # D = 64 (any KV head count)
    (4, 32, 8, 1, 4096 + 64 * 3 + 5, 128, False, 7),
], ids=lambda s: "x".join(map(str, s)))
def test_splitkv_partials_rotated_walk(shape):
    """Workgroups of these shapes start their walk over the split's tiles at a tile that
    depends on (batch, split) and wrap around; each split's partials still equal the oracle's
    for that split's key range."""
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, Lq, Lk, D, causal, splits = shape
    say(f"partials, rotated walk {shape}")
    seed = 8150 + Lk
    q = randn_bf16((B, Lq, Hq, D), seed)
    k = randn_bf16((B, Lk, Hkv, D), seed + 1)
    v = randn_bf16((B, Lk, Hkv, D), seed + 2)
    op = torch.full((splits, B, Hq, Lq, D), float("nan"), dtype=torch.float32, device=DEV)
    lp = torch.full((splits, B, Hq, Lq), float("nan"), dtype=torch.float32, device=DEV)
    S.attn_fwd_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), op, lp, causal=causal, scale=D ** -0.5)
    torch.cuda.synchronize()
    op_ref, lp_ref = A.splitkv_partials(to_f64(q), to_f64(k), to_f64(v),
                                        A.effective_scale(D ** -0.5), causal, splits)
    check_parity(to_f64(op), op_ref, to_f64(lp), lp_ref, f"rotated walk {shape}")
    o, lse = _decode(q.to(DEV), k.to(DEV), v.to(DEV), causal, D ** -0.5, num_splits=splits)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5),
                                 causal)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"rotated walk, combined {shape}")


DECODE_SHAPES = [
    # B, Hq, Hkv, Lq, Lk, Dqk, Dv, causal
    (2, 8, 8, 1, 1000, 128, 128, False),    # MHA, ragged Lk
    (4, 32, 8, 1, 333, 64, 64, False),      # D=64
    (1, 16, 4, 2, 777, 128, 128, True),     # Lq = 2, bottom-right causal, 8 columns
    (1, 16, 1, 2, 1500, 576, 512, True),    # MLA with two query tokens: 32 columns
    (2, 4, 1, 3, 200, 64, 64, True),        # g*Lq = 12 columns
    (1, 40, 2, 1, 130, 128, 128, False),    # g = 20 > 16: two column blocks
]


@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_decode_shapes(shape):
    B, Hq, Hkv, Lq, Lk, Dqk, Dv, causal = shape
    say(f"decode {shape}")
    seed = 8200 + sum(shape)
    q = randn_bf16((B, Lq, Hq, Dqk), seed)
    k = randn_bf16((B, Lk, Hkv, Dqk), seed + 1)
    scale = 1.0 / np.sqrt(192.0 if Dqk == 576 else Dqk)
    if Dqk == 576:
        kd = k.to(DEV)
        vd = kd[..., :512]
        vf = A.mla_value_view(to_f64(k), 512)
    else:
        v = randn_bf16((B, Lk, Hkv, Dv), seed + 2)
        vd = v.to(DEV)
        kd = k.to(DEV)
        vf = to_f64(v)
    o, lse = _decode(q.to(DEV), kd, vd, causal, scale)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), vf, A.effective_scale(scale), causal)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"decode{shape}")


def test_decode_causal_flag_is_noop_for_single_query():
    """With Lq = 1 and bottom-right alignment the query sees every key: causal=1 == causal=0."""
    import torch
    say("decode causal no-op")
    q = randn_bf16((2, 1, 8, 128), 8300)
    k = randn_bf16((2, 500, 2, 128), 8301)
    v = randn_bf16((2, 500, 2, 128), 8302)
    o0, l0 = _decode(q.to(DEV), k.to(DEV), v.to(DEV), False, 0.09)
    o1, l1 = _decode(q.to(DEV), k.to(DEV), v.to(DEV), True, 0.09)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


@pytest.mark.parametrize("Sx,Dv", [(5, 512), (100, 512), (77, 128), (3, 64), (2, 128), (8, 128), (9, 64)])
def test_combine_alone_against_oracle(Sx, Dv):
    """Random partials with empty splits (LSE = -inf), an all-empty row, and rows whose split
    LSEs rise or fall with the split index (so a later pass of one split group moves its
    running maximum)."""
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Lq = 2, 3, 2
    say(f"combine alone S={Sx} Dv={Dv}")
    g = torch.Generator().manual_seed(8400 + Sx)
    op = torch.randn((Sx, B, Hq, Lq, Dv), generator=g, dtype=torch.float32)
    lp = torch.randn((Sx, B, Hq, Lq), generator=g, dtype=torch.float32) * 3
    lp[:, 0, 1, 0] = torch.arange(Sx, dtype=torch.float32) * 0.5
    lp[:, 1, 0, 1] = -torch.arange(Sx, dtype=torch.float32) * 0.5
    lp[1, 0, 0, 0] = -float("inf")
    lp[:, 1, 2, 1] = -float("inf")
    op[:, 1, 2, 1] = 0.0
    o = torch.empty((B, Lq, Hq, Dv), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    S.attn_combine_lse(op.to(DEV), lp.to(DEV), o, lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.combine_lse(op.numpy().astype(np.float64), lp.numpy().astype(np.float64))
    check_parity(to_f64(o), np.transpose(o_ref, (0, 2, 1, 3)), to_f64(lse), lse_ref, "combine")


def test_decode_deterministic():
    say("determinism decode")
    q = randn_bf16((4, 1, 16, 576), 8500)
    k = randn_bf16((4, 3000, 1, 576), 8501).to(DEV)
    o1, l1 = _decode(q.to(DEV), k, k[..., :512], False, 192 ** -0.5)
    o2, l2 = _decode(q.to(DEV), k, k[..., :512], False, 192 ** -0.5)
    assert bool((o1 == o2).all()) and bool((l1 == l2).all())


# ---- the FlashMLA-ETAP decode grid (MLA, 16 heads of dimension 576, one or two query tokens,
# bottom-right causal): with two tokens the 32 query columns share one workgroup, so every
# read of the latent cache feeds both 16-column MFMA blocks.

def _etap(B, Lq, Lk, num_splits=None):
    w = ETAP_GRID["etap_b16_q2_k512"]      # the grid's recipe at reduced sizes
    q, k, _ = make_qkv(w, b=B, lq=Lq, lk=Lk)
    kd = k.to(DEV)
    o, lse = _decode(q.to(DEV), kd, kd[..., :512], True, w.scale, num_splits=num_splits)
    kf = to_f64(k)
    o_ref, lse_ref = A.attention(to_f64(q), kf, A.mla_value_view(kf, 512),
                                 A.effective_scale(w.scale), True)
    return o, lse, o_ref, lse_ref


@pytest.mark.parametrize("shape", [(3, 2, 513), (3, 2, 2049), (3, 1, 2049), (2, 2, 40)],
                         ids=lambda s: "x".join(map(str, s)))
def test_etap_grid_reduced(shape):
    B, Lq, Lk = shape
    say(f"etap reduced B={B} Lq={Lq} Lk={Lk}")
    o, lse, o_ref, lse_ref = _etap(B, Lq, Lk)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"etap{shape}")


@pytest.mark.parametrize("splits", [1, 3, 8, 47])
def test_etap_split_invariance(splits):
    say(f"etap split invariance S={splits}")
    o, lse, o_ref, lse_ref = _etap(2, 2, 3000, num_splits=splits)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"etap splits={splits}")


def test_etap_grid_point_full():
    """A full grid point (batch 16, two query tokens, 16K keys), every output element."""
    w = ETAP_GRID["etap_b16_q2_k16384"]
    say(f"etap full {w}")
    q, k, _ = make_qkv(w)
    kd = k.to(DEV)
    o, lse = _decode(q.to(DEV), kd, kd[..., :512], True, w.scale)
    kf = to_f64(k)
    o_ref, lse_ref = A.attention(to_f64(q), kf, A.mla_value_view(kf, 512),
                                 A.effective_scale(w.scale), True)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, "etap_b16_q2_k16384")


def test_peaky_gqa_decode():
    """Config-3 shape with Q x 4 (concentrated attention) through split-KV + combine."""
    import torch
    w = WORKLOADS["gqa_decode_4k"]
    say("peaky gqa_decode_4k")
    q, k, v = make_qkv(w)
    q = (q.float() * 4.0).to(torch.bfloat16)
    o, lse = _decode(q.to(DEV), k.to(DEV), v.to(DEV), False, w.scale)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(w.scale), False)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, "peaky gqa_decode_4k")

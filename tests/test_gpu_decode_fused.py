"""GPU parity of the one-call decode (attn_fwd_decode: split-KV then the LSE combine, with the
partials in the caller's workspace) against the fp64 oracle, through the C ABI; one workspace
serves calls of several shapes."""

import numpy as np
import pytest

from oracle import attention as A
from tests.helpers import check_parity, say, to_f64
from workloads import WORKLOADS, make_qkv, randn_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(q, k, v, causal, scale, ws=None):
    import torch
    import sparse_attention_attn_amd as S
    B, Lq, Hq, _ = q.shape
    o = torch.empty((B, Lq, Hq, v.shape[3]), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    S.attn_fwd_decode(q, k, v, o, lse, causal=causal, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    return o, lse


def _check(q, k, v, causal, scale, label, ws=None, mla=False, record=None):
    kd = k.to(DEV)
    o, lse = _run(q.to(DEV), kd, kd[..., :512] if mla else v.to(DEV), causal, scale, ws)
    vf = A.mla_value_view(to_f64(k), 512) if mla else to_f64(v)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), vf, A.effective_scale(scale), causal)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, label, record=record)


def _splits(q, k, v):
    import sparse_attention_attn_amd as S
    B, Lq, Hq, Dqk = q.shape
    return S.attn_splitkv_num_splits(B, Hq, k.shape[2], Lq, k.shape[1], Dqk, v.shape[3])


def test_decode_one_call_gqa_workload():
    """The batched GQA decode workload at full size, through the call the bench times."""
    w = WORKLOADS["gqa_decode_4k"]
    say(f"one-call decode {w.name}")
    q, k, v = make_qkv(w)
    _check(q, k, v, False, w.scale, "one-call gqa_decode_4k", record="gqa_decode_4k")


def test_decode_one_call_mla_workload():
    """The MLA decode workload at full size (B 8, 16 heads, 65536 latent keys), through the
    call the bench times."""
    w = WORKLOADS["mla_decode_64k"]
    say(f"one-call decode {w.name}")
    q, k, _ = make_qkv(w)
    _check(q, k, None, False, w.scale, "one-call mla_decode_64k", mla=True,
           record="mla_decode_64k")


@pytest.mark.parametrize("shape", [(1, 16, 1, 2, 200, 576, 512, True),
                                   (64, 8, 4, 1, 300, 64, 64, False)],
                         ids=["mla_lq2_two_colblocks", "d64"])
def test_decode_one_call_direct_path(shape):
    """One split: the split kernel writes O and LSE itself. The MLA shape with two query tokens
    (32 query columns, two 16-column blocks writing O) and D = 64 reach that path too."""
    B, Hq, Hkv, Lq, Lk, Dqk, Dv, causal = shape
    say(f"one-call decode direct {shape}")
    q = randn_bf16((B, Lq, Hq, Dqk), 8800 + Dqk)
    k = randn_bf16((B, Lk, Hkv, Dqk), 8801 + Dqk)
    mla = Dqk == 576
    v = None if mla else randn_bf16((B, Lk, Hkv, Dv), 8802 + Dqk)
    assert _splits(q, k, k[..., :512] if mla else v) == 1
    _check(q, k, v, causal, (192 if mla else Dqk) ** -0.5, f"direct {shape}", mla=mla)


SHAPES = [
    # B, Hq, Hkv, Lq, Lk, D, causal
    (1, 4, 1, 1, 1, 128, False),        # one key, one split
    (3, 8, 2, 1, 4096 + 37, 128, False),
    (2, 16, 4, 2, 3000, 128, True),     # two query tokens, bottom-right causal
    (5, 8, 8, 1, 777, 64, False),
    (2, 6, 2, 3, 2049, 64, True),
    (2, 16, 4, 2, 300, 128, True),      # short splits: 128, 128 and 44 keys
    (2, 16, 4, 2, 100, 128, True),      # one split (under 128 keys): O and LSE written directly
    (128, 32, 8, 1, 1024, 128, False),  # one split (1024 units fill the GPU): direct too
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_decode_one_call_shapes(shape):
    B, Hq, Hkv, Lq, Lk, D, causal = shape
    say(f"one-call decode {shape}")
    q = randn_bf16((B, Lq, Hq, D), 8600 + Lk)
    k = randn_bf16((B, Lk, Hkv, D), 8601 + Lk)
    v = randn_bf16((B, Lk, Hkv, D), 8602 + Lk)
    _check(q, k, v, causal, D ** -0.5, f"one-call {shape}")


def test_decode_one_call_mla():
    """The latent shape takes the two-launch path inside the same entry point."""
    B, Hq, Lk = 2, 16, 5000
    say("one-call decode MLA")
    q = randn_bf16((B, 1, Hq, 576), 8700)
    k = randn_bf16((B, Lk, 1, 576), 8701)
    _check(q, k, None, False, 192 ** -0.5, "one-call MLA", mla=True)


def test_workspace_reuse_across_shapes():
    """One workspace, sized for the largest shape and filled with garbage, serves calls of
    several shapes in a row."""
    import torch
    import sparse_attention_attn_amd as S
    say("one-call decode workspace reuse")
    shapes = [(4, 32, 8, 1, 4096, 128), (2, 8, 2, 2, 1500, 64), (4, 32, 8, 1, 4096, 128),
              (1, 4, 4, 1, 100, 128)]
    need = max(S.attn_decode_workspace_bytes(B, Hq, Hkv, Lq, Lk, D, D)
               for B, Hq, Hkv, Lq, Lk, D in shapes)
    ws = torch.full((need,), 0x7f, dtype=torch.uint8, device=DEV)
    for i, (B, Hq, Hkv, Lq, Lk, D) in enumerate(shapes):
        q = randn_bf16((B, Lq, Hq, D), 8800 + i)
        k = randn_bf16((B, Lk, Hkv, D), 8810 + i)
        v = randn_bf16((B, Lk, Hkv, D), 8820 + i)
        _check(q, k, v, Lq > 1, D ** -0.5, f"reuse {i}", ws=ws)


def test_decode_one_call_deterministic():
    import torch
    say("one-call decode determinism")
    q = randn_bf16((8, 1, 32, 128), 8900).to(DEV)
    k = randn_bf16((8, 3000, 8, 128), 8901).to(DEV)
    v = randn_bf16((8, 3000, 8, 128), 8902).to(DEV)
    a = _run(q, k, v, False, 0.088)
    b = _run(q, k, v, False, 0.088)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_one_call_mla_one_split():
    """The MLA latent shape with one split (250 keys): the split kernel writes O and LSE."""
    import sparse_attention_attn_amd as S
    B, Hq, Lq, Lk = 2, 16, 1, 250
    say("one-call MLA decode, one split")
    assert S.attn_splitkv_num_splits(B, Hq, 1, Lq, Lk, 576, 512) == 1
    q = randn_bf16((B, Lq, Hq, 576), 8700)
    k = randn_bf16((B, Lk, 1, 576), 8701)
    _check(q, k, None, True, 192 ** -0.5, "one-call MLA one split", mla=True)


def test_decode_one_split_equals_partials_path():
    """One split through attn_fwd_decode (direct outputs) equals attn_fwd_splitkv with one split
    followed by attn_combine_lse, bit for bit."""
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, Lq, Lk, D = 128, 16, 4, 2, 300, 128   # 512 (b, KV head) units: one split
    say("one split: direct outputs vs partials + combine")
    q = randn_bf16((B, Lq, Hq, D), 8710).to(DEV)
    k = randn_bf16((B, Lk, Hkv, D), 8711).to(DEV)
    v = randn_bf16((B, Lk, Hkv, D), 8712).to(DEV)
    assert S.attn_splitkv_num_splits(B, Hq, Hkv, Lq, Lk, D, D) == 1
    o1, l1 = _run(q, k, v, True, D ** -0.5)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    S.splitkv_decode(q, k, v, o2, l2, causal=True, scale=D ** -0.5, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("shape", [
    # B, Hq, Hkv, Lq, Lk, Dqk, causal
    (2, 8, 2, 2, 1, 128, True),      # Lq > Lk, bottom-right causal: query row 0 sees no key
    (2, 8, 2, 3, 2, 64, True),       # rows see 0, 1 and 2 keys
    (1, 16, 1, 2, 1, 576, True),     # the latent shape with an empty row
    (3, 8, 8, 1, 63, 128, False),    # one key short of a tile
    (3, 8, 8, 1, 64, 128, False),    # exactly one tile
    (3, 8, 8, 1, 65, 128, False),    # one key into a second tile
    (1, 16, 1, 1, 127, 576, False),  # the latent shape's split minimum, one key short
    (1, 16, 1, 1, 129, 576, False),  # one key past it
    (1, 8, 1, 1, 130, 128, False),   # two splits, the second of 2 keys
    (1, 16, 1, 2, 257, 576, True),   # latent, two splits (192 + 65 keys), two tokens
], ids=lambda s: "x".join(map(str, s)))
def test_decode_edge_lengths(shape):
    """Cache lengths at tile edges and query rows with no visible key (O = 0, LSE = -inf in
    both the kernel and the oracle)."""
    B, Hq, Hkv, Lq, Lk, Dqk, causal = shape
    mla = Dqk == 576
    say(f"decode edge {shape}")
    q = randn_bf16((B, Lq, Hq, Dqk), 8500 + Lk + Lq)
    k = randn_bf16((B, Lk, Hkv, Dqk), 8501 + Lk + Lq)
    v = None if mla else randn_bf16((B, Lk, Hkv, Dqk), 8502 + Lk + Lq)
    _check(q, k, v, causal, (192 if mla else Dqk) ** -0.5, f"decode edge {shape}", mla=mla)

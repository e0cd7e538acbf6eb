"""GPU parity of attn_fwd (dense prefill) against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest

from oracle import attention as A
from tests.helpers import check_parity, say, to_f64
from workloads import WORKLOADS, make_qkv, randn_bf16, sampled_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run_fwd(q, k, v, causal, scale):
    import torch
    import sparse_attention_attn_amd as S
    B, Lq, Hq, _ = q.shape
    o = torch.empty((B, Lq, Hq, v.shape[3]), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    S.attn_fwd(q, k, v, o, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _qkv(B, Hq, Hkv, Lq, Lk, D, seed):
    q = randn_bf16((B, Lq, Hq, D), seed)
    k = randn_bf16((B, Lk, Hkv, D), seed + 1)
    v = randn_bf16((B, Lk, Hkv, D), seed + 2)
    return q, k, v


def test_tiny_causal_workload_full():
    w = WORKLOADS["tiny_causal"]
    say(f"tiny_causal full {w}")
    q, k, v = make_qkv(w)
    o, lse = _run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), True, w.scale)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(w.scale), True)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, "tiny_causal", record="tiny_causal")


SHAPES = [
    # B, Hq, Hkv, Lq, Lk, D, causal
    (1, 4, 2, 200, 200, 128, True),     # ragged: one full 128-row tile + 72
    (2, 8, 2, 333, 333, 64, True),      # GQA g=4, ragged, D=64
    (1, 4, 4, 130, 390, 128, True),     # Lq < Lk: bottom-right causal
    (1, 2, 1, 300, 129, 64, False),     # Lq > Lk non-causal
    (1, 4, 1, 390, 130, 128, True),     # Lq > Lk causal: leading rows see nothing
    (1, 8, 8, 1, 517, 128, True),       # one query row through the prefill path
    (1, 2, 2, 64, 64, 64, True),        # exactly one tile
    (3, 6, 3, 257, 257, 128, False),    # non-causal, ragged, B=3
    (1, 32, 8, 1024, 1024, 128, True),  # several full tiles with the workload's head layout
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_prefill_shapes(shape):
    B, Hq, Hkv, Lq, Lk, D, causal = shape
    say(f"prefill {shape}")
    seed = 7000 + sum(shape)
    q, k, v = _qkv(B, Hq, Hkv, Lq, Lk, D, seed)
    scale = D ** -0.5
    o, lse = _run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal, scale)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(scale), causal)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"prefill{shape}")


def test_prefill_strided_packed_qkv():
    """Q, K, V as views into one packed [B, L, Hq + 2*Hkv, D] buffer; O written into a wider
    buffer: exercises the stride arguments."""
    import torch
    B, Hq, Hkv, L, D = 2, 4, 2, 190, 128
    say(f"prefill packed qkv B={B} Hq={Hq} Hkv={Hkv} L={L} D={D}")
    packed = randn_bf16((B, L, Hq + 2 * Hkv, D), 7100)
    q, k, v = packed[:, :, :Hq], packed[:, :, Hq:Hq + Hkv], packed[:, :, Hq + Hkv:]
    pd = packed.to(DEV)
    qd, kd, vd = pd[:, :, :Hq], pd[:, :, Hq:Hq + Hkv], pd[:, :, Hq + Hkv:]
    obuf = torch.zeros((B, L, Hq + 3, D), dtype=torch.bfloat16, device=DEV)
    od = obuf[:, :, 1:1 + Hq]
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    import sparse_attention_attn_amd as S
    S.attn_fwd(qd, kd, vd, od, lse, causal=True, scale=D ** -0.5)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5), True)
    check_parity(to_f64(od), o_ref, to_f64(lse), lse_ref, "packed")
    # untouched neighbours stay zero
    assert float(obuf[:, :, 0].abs().max()) == 0.0 and float(obuf[:, :, 1 + Hq:].abs().max()) == 0.0


def test_gqa_prefill_8k_full_size_all_rows():
    """The Llama-3-8B-shaped workload at full size, every element of O and LSE (all 8192 rows
    of all 32 query heads) against the fp64 oracle, one head at a time."""
    w = WORKLOADS["gqa_prefill_8k"]
    say(f"gqa_prefill_8k full size {w}")
    q, k, v = make_qkv(w)
    o, lse = _run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), True, w.scale)
    rows = np.arange(w.Lq)
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    of, lf = to_f64(o), to_f64(lse)
    sc = A.effective_scale(w.scale)
    got_o = np.empty((w.Hq, w.Lq, w.Dv))
    ref_o = np.empty((w.Hq, w.Lq, w.Dv))
    ref_l = np.empty((w.Hq, w.Lq))
    for h in range(w.Hq):
        ref_o[h], ref_l[h] = A.attention_rows(qf, kf, vf, sc, True, 0, h, rows)
        got_o[h] = of[0, :, h, :]
    check_parity(got_o, ref_o, lf[0], ref_l, "gqa_8k all rows", record="gqa_prefill_8k")


def test_closed_forms_on_gpu():
    """Causal row 0 returns V_0 exactly; constant V returns the constant; uniform keys give
    prefix means (closed forms of the definition)."""
    import torch
    B, H, L, D = 1, 2, 300, 128
    say("closed forms")
    q = randn_bf16((B, L, H, D), 7200)
    k = randn_bf16((B, L, H, D), 7201)
    v = randn_bf16((B, L, H, D), 7202)
    o, _ = _run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), True, D ** -0.5)
    assert torch.equal(o[:, 0].cpu(), v[:, 0]), "causal row 0 must be V_0 bit-exactly"
    vc = torch.full((B, L, H, D), -1.75, dtype=torch.bfloat16)
    o, _ = _run_fwd(q.to(DEV), k.to(DEV), vc.to(DEV), True, D ** -0.5)
    assert float((o.float() + 1.75).abs().max()) <= 1e-2
    ku = k[:, :1].expand(B, L, H, D).contiguous()
    o, lse = _run_fwd(q.to(DEV), ku.to(DEV), v.to(DEV), True, D ** -0.5)
    n = np.arange(1, L + 1)
    mean = np.cumsum(to_f64(v), axis=1) / n[None, :, None, None]
    check_parity(to_f64(o), mean, label="uniform keys -> prefix means")
    s = A.effective_scale(D ** -0.5) * np.einsum("blhd,bhd->bhl", to_f64(q), to_f64(k[:, 0]))
    assert np.max(np.abs(to_f64(lse) - (s + np.log(n)[None, None, :]))) <= 1e-3


def test_single_key():
    say("Lk = 1")
    q = randn_bf16((2, 5, 4, 64), 7300)
    k = randn_bf16((2, 1, 2, 64), 7301)
    v = randn_bf16((2, 1, 2, 64), 7302)
    o, lse = _run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), False, 0.125)
    expect = v.repeat_interleave(2, dim=2).expand(2, 5, 4, 64)
    assert (o.cpu() == expect).all()


def test_planted_keys_causal_boundary():
    """Keys aligned with a query carry about half the weight: an off-by-one at the causal
    boundary or a dropped tile moves O by far more than the tolerance."""
    import torch
    B, H, L, D = 1, 1, 256, 64
    say("planted keys")
    q = randn_bf16((B, L, H, D), 7400).float()
    k = randn_bf16((B, L, H, D), 7401).float() * 0.1
    v = randn_bf16((B, L, H, D), 7402).float()
    for i in (63, 64, 127, 128, 200):
        k[0, i, 0] = q[0, i, 0] * 0.6   # strong self-match on the diagonal
        v[0, i, 0] = 3.0   # |O| < 4: bf16 output rounding (half-ulp <= 2^-8) stays far inside 1e-2
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    o, lse = _run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), True, D ** -0.5)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5), True)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, "planted")


def test_reference_jumps():
    """Scores that rise by about 29 (exp2 domain) per 32 keys in some heads and fall in others:
    weights against a reference set on early keys overflow fp32 within a few units, so the
    kernel has to move its reference mid-row; falling scores underflow instead."""
    import torch
    B, H, L, D = 1, 4, 256, 64
    say("reference jumps")
    u = torch.full((D,), 1.0)
    t = 20.0 * (torch.arange(L) // 32).float()               # 0, 20, ..., 140
    q = u.expand(B, L, H, D) + 0.1 * randn_bf16((B, L, H, D), 7600).float()
    k = 0.1 * randn_bf16((B, L, H, D), 7601).float()
    k[0, :, 0] += t[:, None] / 8.0                           # rising: s grows by 160 per unit
    k[0, :, 1] += t.flip(0)[:, None] / 8.0                   # falling
    k[0, :, 2] += (t[:, None] / 8.0) * ((torch.arange(L) % 64) < 32).float()[:, None]
    v = randn_bf16((B, L, H, D), 7602).float()
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    scale = D ** -0.5
    for causal in (True, False):
        o, lse = _run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal, scale)
        o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(scale),
                                     causal)
        assert np.isfinite(to_f64(o)).all()
        check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"reference jumps causal={causal}")


def test_prefill_deterministic():
    say("determinism prefill")
    q, k, v = _qkv(1, 8, 2, 700, 700, 128, 7500)
    o1, l1 = _run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), True, 0.088)
    o2, l2 = _run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), True, 0.088)
    assert bool((o1 == o2).all()) and bool((l1 == l2).all())


def _peaky(t):
    """Q scaled by 4 in fp32, then rounded to bf16: scores with 4x the spread, attention that
    concentrates on few keys (exercises the softmax's reference moves and large weights)."""
    import torch
    return (t.float() * 4.0).to(torch.bfloat16)


def test_peaky_tiny_causal():
    w = WORKLOADS["tiny_causal"]
    say("peaky tiny_causal")
    q, k, v = make_qkv(w)
    q = _peaky(q)
    o, lse = _run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), True, w.scale)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(w.scale), True)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, "peaky tiny")


def test_peaky_gqa_prefill_8k_sampled_rows():
    """Config-2 shape with Q x 4, 96 sampled rows of every query head."""
    w = WORKLOADS["gqa_prefill_8k"]
    say("peaky gqa_prefill_8k")
    q, k, v = make_qkv(w)
    q = _peaky(q)
    o, lse = _run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), True, w.scale)
    rows = sampled_rows(w.Lq, 96, 1000 * w.index + 5, edge=32)
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    of, lf = to_f64(o), to_f64(lse)
    sc = A.effective_scale(w.scale)
    got_o, ref_o, got_l, ref_l = [], [], [], []
    for h in range(w.Hq):
        orow, lrow = A.attention_rows(qf, kf, vf, sc, True, 0, h, rows)
        got_o.append(of[0, rows, h, :])
        ref_o.append(orow)
        got_l.append(lf[0, h, rows])
        ref_l.append(lrow)
    check_parity(np.stack(got_o), np.stack(ref_o), np.stack(got_l), np.stack(ref_l), "peaky 8k")


@pytest.mark.parametrize("shape", [(3, 8, 1, 1100), (5, 4, 1, 2000), (3, 4, 2, 2000),
                                   (3, 8, 4, 1100), (1, 12, 3, 2048), (2, 16, 8, 1300)],
                         ids=lambda s: "x".join(map(str, s)))
def test_prefill_xcd_group_counts(shape):
    """Batch x KV-head group counts of 3, 5, 6, 12, 3 and 16: every one of the launcher's XCD
    cluster sizes (8 / gcd(groups, 8)) places all tiles exactly once (element-by-element parity
    over every row of every head)."""
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, L = shape
    D = 128
    say(f"prefill XCD placement {shape}: {B * Hkv} groups")
    q = randn_bf16((B, L, Hq, D), 9900 + B * Hkv)
    k = randn_bf16((B, L, Hkv, D), 9901 + B * Hkv)
    v = randn_bf16((B, L, Hkv, D), 9902 + B * Hkv)
    o = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    S.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), o, lse, causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5),
                               True)
    check_parity(to_f64(o), o_ref, to_f64(lse), l_ref, f"prefill groups {shape}")

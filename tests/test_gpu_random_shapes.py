"""Seeded sweep of random shapes through every forward entry point, each checked against the
fp64 oracle element by element: dense prefill (attn_fwd), decode (attn_fwd_decode, GQA and the
MLA latent shape), chunked prefill (attn_fwd_decode over query chunks of 64 to 700 rows),
block-sparse (attn_fwd_blocksparse) and vertical-slash (attn_fwd_vertical_slash) over random
lists. The shapes mix batch sizes, GQA ratios, ragged
and tile-aligned lengths, Lq above and below Lk, D = 64 and 128, causal and not, so that the
combinations the hand-picked cases do not list are covered too. Sizes stay small enough for
the oracle to finish each case in well under a second."""

import numpy as np
import pytest

from oracle import attention as A
from tests.helpers import check_parity, say, to_f64
from workloads import randn_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_CASES = 12


def _shape(rng, lmax=700):
    B = int(rng.integers(1, 4))
    Hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    # a third of the lengths are multiples of 64 (whole tiles), the rest ragged
    def length():
        n = int(rng.integers(1, lmax))
        return max(64, n - n % 64) if rng.random() < 0.33 else n
    return B, Hkv * g, Hkv, length(), length(), D, bool(rng.random() < 0.7)


def _qkv(B, Hq, Hkv, Lq, Lk, D, seed, Dv=None):
    Dv = D if Dv is None else Dv
    return (randn_bf16((B, Lq, Hq, D), seed), randn_bf16((B, Lk, Hkv, D), seed + 1),
            randn_bf16((B, Lk, Hkv, Dv), seed + 2))


def _outs(B, Lq, Hq, Dv):
    import torch
    return (torch.empty((B, Lq, Hq, Dv), dtype=torch.bfloat16, device=DEV),
            torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_prefill(case):
    import torch
    import sparse_attention_attn_amd as S
    rng = np.random.default_rng(100 + case)
    B, Hq, Hkv, Lq, Lk, D, causal = _shape(rng)
    scale = float(rng.choice([1.0, -1.0])) * D ** -0.5 * float(rng.uniform(0.5, 2.0))
    say(f"random prefill {case}: B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D} causal={causal} "
        f"scale={scale:.4f}")
    q, k, v = _qkv(B, Hq, Hkv, Lq, Lk, D, 20000 + 10 * case)
    o, lse = _outs(B, Lq, Hq, D)
    S.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), o, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(scale),
                                 causal)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"random prefill {case}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_decode(case):
    import torch
    import sparse_attention_attn_amd as S
    rng = np.random.default_rng(200 + case)
    mla = case % 3 == 2
    B = int(rng.integers(1, 5))
    Lq = int(rng.choice([1, 2]))
    Lk = int(rng.integers(1, 5000))
    causal = bool(rng.random() < 0.5) or Lq > Lk
    if mla:
        Hq, Hkv, Dqk, Dv = 16, 1, 576, 512
    else:
        Hkv = int(rng.choice([1, 2, 4, 8]))
        Hq, Dqk = Hkv * int(rng.choice([1, 2, 4, 8])), int(rng.choice([64, 128]))
        Dv = Dqk
    scale = Dqk ** -0.5 if not mla else 192 ** -0.5
    say(f"random decode {case}: B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{Dqk}/{Dv} causal={causal}")
    q = randn_bf16((B, Lq, Hq, Dqk), 21000 + 10 * case)
    k = randn_bf16((B, Lk, Hkv, Dqk), 21001 + 10 * case)
    if mla:
        kd = k.to(DEV)
        vd = kd[..., :Dv]
        v_ref = A.mla_value_view(to_f64(k), Dv)
    else:
        v = randn_bf16((B, Lk, Hkv, Dv), 21002 + 10 * case)
        kd, vd, v_ref = k.to(DEV), v.to(DEV), to_f64(v)
    o, lse = _outs(B, Lq, Hq, Dv)
    S.attn_fwd_decode(q.to(DEV), kd, vd, o, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), v_ref, A.effective_scale(scale), causal)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"random decode {case}")


def _csr(per_row):
    ptr, parts = [0], []
    for x in per_row:
        x = np.asarray(sorted(set(int(t) for t in x)), np.int32)
        parts.append(x)
        ptr.append(ptr[-1] + x.size)
    idx = np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)
    return np.asarray(ptr, np.int32), idx


def _random_lists(rng, B, Hq, Lq, Lk):
    nqb, nkb = -(-Lq // 64), -(-Lk // 64)
    blocks = [rng.choice(nkb, int(rng.integers(0, min(nkb, 6) + 1)), replace=False).tolist()
              for _ in range(B * Hq * nqb)]
    cols = [rng.choice(Lk, int(rng.integers(0, min(Lk, 40) + 1)), replace=False).tolist()
            for _ in range(B * Hq)]
    return _csr(blocks) + _csr(cols)


def _dev(x):
    import torch
    return torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32)).to(DEV)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_blocksparse(case):
    import torch
    import sparse_attention_attn_amd as S
    rng = np.random.default_rng(300 + case)
    B, Hq, Hkv, Lq, Lk, D, causal = _shape(rng, lmax=900)
    say(f"random block-sparse {case}: B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D} causal={causal}")
    q, k, v = _qkv(B, Hq, Hkv, Lq, Lk, D, 22000 + 10 * case)
    bp, bi, cp, ci = _random_lists(rng, B, Hq, Lq, Lk)
    S.attn_blocksparse_check(bp, bi, cp, ci, B, Hq, Lq, Lk)
    o, lse = _outs(B, Lq, Hq, D)
    S.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), o, _dev(bp), _dev(bi), _dev(cp),
                           _dev(ci), lse=lse, causal=causal)
    torch.cuda.synchronize()
    fn = A.csr_allowed_fn(bp, bi, cp, ci, hq=Hq, nqb=-(-Lq // 64), lk=Lk)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5),
                                 causal, allowed_fn=fn)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"random block-sparse {case}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_vertical_slash(case):
    import torch
    import sparse_attention_attn_amd as S
    rng = np.random.default_rng(400 + case)
    B, Hq, Hkv, Lq, Lk, D, _ = _shape(rng, lmax=900)
    say(f"random vertical-slash {case}: B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D}")
    q, k, v = _qkv(B, Hq, Hkv, Lq, Lk, D, 23000 + 10 * case)
    bp, bi, cp, ci = _random_lists(rng, B, Hq, Lq, Lk)
    # per head: a run of offsets from 0 (its width random, up to 200), a few short runs and
    # isolated offsets elsewhere
    slashes = []
    for _ in range(B * Hq):
        offs = list(range(int(rng.integers(0, 200))))
        for _r in range(int(rng.integers(0, 3))):
            s0 = int(rng.integers(0, Lk))
            offs += list(range(s0, min(Lk, s0 + int(rng.integers(2, 6)))))
        offs += rng.choice(Lk, min(Lk, int(rng.integers(0, 12))), replace=False).tolist()
        slashes.append([o for o in offs if o < Lk])
    sp, si = _csr(slashes)
    S.attn_blocksparse_check(bp, bi, cp, ci, B, Hq, Lq, Lk)
    S.attn_vertical_slash_check(sp, si, B, Hq, Lk)
    o, lse = _outs(B, Lq, Hq, D)
    S.attn_fwd_vertical_slash(q.to(DEV), k.to(DEV), v.to(DEV), o, _dev(bp), _dev(bi), _dev(cp),
                              _dev(ci), _dev(sp), _dev(si), lse=lse, causal=True)
    torch.cuda.synchronize()
    fn = A.vslash_allowed_fn(bp, bi, cp, ci, sp, si, Hq, -(-Lq // 64), Lq, Lk)
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5),
                                 True, allowed_fn=fn)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"random vertical-slash {case}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_chunked_prefill(case):
    """A random query chunk against a longer cache through the one-call split path
    (attn_fwd_decode): 64 to 700 query rows over up to 12000 keys, so both the prefill kernel's
    split form and, for the shorter chunks over short caches, the decode kernel are drawn."""
    import torch
    import sparse_attention_attn_amd as S
    rng = np.random.default_rng(500 + case)
    B = int(rng.integers(1, 3))
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    Lq = int(rng.integers(64, 701))
    Lk = int(rng.integers(Lq, 12001))
    causal = bool(rng.random() < 0.7)
    nsp = S.attn_splitkv_num_splits(B, Hq, Hkv, Lq, Lk, D, D)
    say(f"random chunked prefill {case}: B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D} "
        f"causal={causal}, {nsp} splits")
    q, k, v = _qkv(B, Hq, Hkv, Lq, Lk, D, 24000 + 10 * case)
    o, lse = _outs(B, Lq, Hq, D)
    S.attn_fwd_decode(q.to(DEV), k.to(DEV), v.to(DEV), o, lse, causal=causal, scale=D ** -0.5)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.attention(to_f64(q), to_f64(k), to_f64(v), A.effective_scale(D ** -0.5),
                                 causal)
    check_parity(to_f64(o), o_ref, to_f64(lse), lse_ref, f"random chunked prefill {case}")

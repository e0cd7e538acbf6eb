"""GPU parity at the largest supported sizes, on sampled query rows against the fp64 oracle:
block-sparse at 2^20 keys (its limit), vertical-slash at 2^19 keys (its limit), a dense causal
prefill of 2^17 tokens, and split-KV decode over 2^20 cached keys (GQA and the MLA latent)."""

import numpy as np
import pytest

from oracle import attention as A
from tests.helpers import check_parity, say, to_f64
from workloads import randn_bf16_device, sampled_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dev(x):
    import torch
    return torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32)).to(DEV)


def _lists(B, Hq, L, seed, extra=2, ncols=64):
    """Per query block: block 0, the diagonal block and the one before it, and `extra` random
    causal blocks; per head `ncols` random columns. CSR int32, sorted and unique."""
    rng = np.random.default_rng(seed)
    nqb = -(-L // 64)
    ptr, idx = [0], []
    for _ in range(B * Hq):
        for qb in range(nqb):
            blks = {0, qb, max(qb - 1, 0)}
            blks.update(int(x) for x in rng.integers(0, qb + 1, extra))
            b = sorted(blks)
            idx.extend(b)
            ptr.append(ptr[-1] + len(b))
    cptr, cidx = [0], []
    for _ in range(B * Hq):
        c = np.unique(rng.integers(0, L, ncols))
        cidx.extend(int(x) for x in c)
        cptr.append(cptr[-1] + c.size)
    return (np.asarray(ptr, np.int32), np.asarray(idx, np.int32), np.asarray(cptr, np.int32),
            np.asarray(cidx, np.int32))


def _check_rows(q, k, v, rows, o, lse, keys_of, causal, scale, label):
    """keys_of(h, row) -> sorted candidate keys of that row (the mask restricted to them)."""
    Hq, Hkv = q.shape[2], k.shape[2]
    g = Hq // Hkv
    Lq, Lk = q.shape[1], k.shape[1]
    go, ro, gl, rl = [], [], [], []
    for h in range(Hq):
        kh = k[0, :, h // g].double().numpy()
        vh = v[0, :, h // g].double().numpy()
        for r in rows:
            orow, lrow = A.attention_rows_over_keys(q[0, [r], h].double().numpy(), [r], kh, vh,
                                                    A.effective_scale(scale), keys_of(h, r), Lq,
                                                    Lk, causal)
            go.append(o[[r], h])
            ro.append(orow)
            gl.append(lse[h, [r]])
            rl.append(lrow)
    check_parity(np.concatenate(go), np.concatenate(ro), np.concatenate(gl), np.concatenate(rl),
                 label)


def _inputs(B, Lq, Lk, Hq, Hkv, Dqk, Dv, seed):
    q = randn_bf16_device((B, Lq, Hq, Dqk), seed)
    k = randn_bf16_device((B, Lk, Hkv, Dqk), seed + 1)
    v = randn_bf16_device((B, Lk, Hkv, Dv), seed + 2)
    return q, k, v


def test_blocksparse_max_keys():
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, L, D = 1, 2, 1, 1 << 20, 128
    say(f"blocksparse at the key limit L={L}")
    q, k, v = _inputs(B, L, L, Hq, Hkv, D, D, 9910)
    bp, bi, cp, ci = _lists(B, Hq, L, 9913)
    S.attn_blocksparse_check(bp, bi, cp, ci, B, Hq, L, L)
    o = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    S.attn_fwd_blocksparse(q, k, v, o, _dev(bp), _dev(bi), _dev(cp), _dev(ci), lse=lse,
                           causal=True, scale=D ** -0.5)
    torch.cuda.synchronize()
    rows = sampled_rows(L, 192, 9914, edge=32)
    nqb = L // 64
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()

    def keys_of(h, r):
        qb = r // 64
        return A.blocksparse_keys(bi[bp[h * nqb + qb]:bp[h * nqb + qb + 1]], ci[cp[h]:cp[h + 1]], L)

    _check_rows(qc, kc, vc, rows, to_f64(o[0].cpu()), lse[0].cpu().numpy(), keys_of, True,
                D ** -0.5, f"blocksparse L={L}")


def test_vslash_max_keys():
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, L, D = 1, 2, 1, 1 << 19, 128
    say(f"vertical-slash at the key limit L={L}")
    q, k, v = _inputs(B, L, L, Hq, Hkv, D, D, 9920)
    bp, bi, cp, ci = _lists(B, Hq, L, 9923, extra=1, ncols=40)
    rng = np.random.default_rng(9924)
    offs = [np.unique(np.concatenate([np.arange(0, 16), rng.integers(16, L, 8)]))
            for _ in range(B * Hq)]
    sp = np.asarray([0] + list(np.cumsum([x.size for x in offs])), np.int32)
    si = np.concatenate(offs).astype(np.int32)
    S.attn_vertical_slash_check(sp, si, B, Hq, L)
    o = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    S.attn_fwd_vertical_slash(q, k, v, o, _dev(bp), _dev(bi), _dev(cp), _dev(ci), _dev(sp),
                              _dev(si), lse=lse, causal=True, scale=D ** -0.5)
    torch.cuda.synchronize()
    rows = sampled_rows(L, 128, 9925, edge=32)
    nqb = L // 64
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()

    def keys_of(h, r):
        qb = r // 64
        base = A.blocksparse_keys(bi[bp[h * nqb + qb]:bp[h * nqb + qb + 1]], ci[cp[h]:cp[h + 1]], L)
        diag = np.nonzero(A.slash_row_mask([r], L, L, si[sp[h]:sp[h + 1]])[0])[0]
        return np.union1d(base, diag)

    _check_rows(qc, kc, vc, rows, to_f64(o[0].cpu()), lse[0].cpu().numpy(), keys_of, True,
                D ** -0.5, f"vslash L={L}")


def test_dense_long_context():
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, L, D = 1, 2, 1, 1 << 17, 128
    say(f"dense causal prefill L={L}")
    q, k, v = _inputs(B, L, L, Hq, Hkv, D, D, 9930)
    o = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    S.attn_fwd(q, k, v, o, lse, causal=True, scale=D ** -0.5)
    torch.cuda.synchronize()
    rows = sampled_rows(L, 64, 9931, edge=8)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    of, lf = to_f64(o[0].cpu()), lse[0].cpu().numpy()
    go, ro, gl, rl = [], [], [], []
    for h in range(Hq):  # every key is a candidate: one oracle call per head for all rows
        orow, lrow = A.attention_rows_over_keys(qc[0, rows, h].double().numpy(), rows,
                                                kc[0, :, 0].double().numpy(),
                                                vc[0, :, 0].double().numpy(),
                                                A.effective_scale(D ** -0.5), np.arange(L), L, L,
                                                True)
        go.append(of[rows, h])
        ro.append(orow)
        gl.append(lf[h, rows])
        rl.append(lrow)
    check_parity(np.concatenate(go), np.concatenate(ro), np.concatenate(gl), np.concatenate(rl),
                 f"dense L={L}")


@pytest.mark.parametrize("mla", [False, True], ids=["gqa", "mla"])
def test_decode_long_context(mla):
    import torch
    import sparse_attention_attn_amd as S
    Lk = 1 << 20
    if mla:
        B, Hq, Hkv, Dqk, Dv, scale = 1, 16, 1, 576, 512, 192 ** -0.5
    else:
        B, Hq, Hkv, Dqk, Dv, scale = 1, 8, 1, 128, 128, 128 ** -0.5
    say(f"decode over {Lk} keys mla={mla}")
    q, k, v = _inputs(B, 1, Lk, Hq, Hkv, Dqk, Dv, 9940 + int(mla))
    vd = k[..., :512] if mla else v
    o = torch.empty((B, 1, Hq, Dv), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=DEV)
    S.splitkv_decode(q, k, vd, o, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    kf = to_f64(k.cpu())
    vf = A.mla_value_view(kf, 512) if mla else to_f64(v.cpu())
    o_ref, lse_ref = A.attention(to_f64(q.cpu()), kf, vf, A.effective_scale(scale), True)
    check_parity(to_f64(o.cpu()), o_ref, to_f64(lse.cpu()), lse_ref, f"decode Lk={Lk}")

"""GPU parity on tensors of more than 2^32 bytes, so that every byte offset the kernels form
past 4 GiB (batch and row strides times large indices) is exercised: a dense causal GQA prefill
whose Q and O hold 4.3 GB each, a split-KV decode whose K and V hold 4.3 GB each, and a
block-sparse prefill on the prefill's tensors. The lengths are ragged (not whole 64-key tiles).
Checked against the fp64 oracle on sampled query rows of the first and the last batch entry,
whose rows lie at the smallest and the largest offsets."""

import numpy as np
import pytest

from oracle import attention as A
from tests.helpers import check_parity, say, to_f64
from workloads import randn_bf16_device, sampled_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GIB4 = 1 << 32


def _nbytes(t):
    return t.numel() * t.element_size()


def _check_rows(q, k, v, o, lse, b, heads, rows, keys_of, causal, scale, label):
    """Oracle rows of batch entry b. keys_of(h, r) gives the keys row r of head h may see; None
    means every key (then one oracle call per head covers all rows)."""
    Hq, Hkv = q.shape[2], k.shape[2]
    g = Hq // Hkv
    Lq, Lk = q.shape[1], k.shape[1]
    rows = np.asarray(rows, dtype=np.int64)
    go, ro, gl, rl = [], [], [], []
    for h in heads:
        qh = q[b, :, h][rows].cpu().double().numpy()
        kh = k[b, :, h // g].cpu().double().numpy()
        vh = v[b, :, h // g].cpu().double().numpy()
        if keys_of is None:
            orow, lrow = A.attention_rows_over_keys(qh, rows, kh, vh, A.effective_scale(scale),
                                                    np.arange(Lk), Lq, Lk, causal)
            ro.append(orow)
            rl.append(lrow)
        else:
            for i, r in enumerate(rows):
                orow, lrow = A.attention_rows_over_keys(qh[[i]], [r], kh, vh,
                                                        A.effective_scale(scale), keys_of(h, r),
                                                        Lq, Lk, causal)
                ro.append(orow)
                rl.append(lrow)
        go.append(to_f64(o[b, :, h][rows].cpu()))
        gl.append(lse[b, h][rows].cpu().numpy())
    check_parity(np.concatenate(go), np.concatenate(ro), np.concatenate(gl), np.concatenate(rl),
                 label)


def _prefill_inputs():
    import torch
    B, L, Hq, Hkv, D = 4, 66000, 64, 8, 128
    q = randn_bf16_device((B, L, Hq, D), 9950)
    k = randn_bf16_device((B, L, Hkv, D), 9951)
    v = randn_bf16_device((B, L, Hkv, D), 9952)
    o = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    assert _nbytes(q) > GIB4 and _nbytes(o) > GIB4
    return q, k, v, o, lse


def test_prefill_beyond_4gib():
    import torch
    import sparse_attention_attn_amd as S
    q, k, v, o, lse = _prefill_inputs()
    B, L, Hq, D = q.shape
    say(f"dense causal prefill B{B} L{L} Hq{Hq}: Q and O {_nbytes(q) / 1e9:.2f} GB each")
    S.attn_fwd(q, k, v, o, lse, causal=True, scale=D ** -0.5)
    torch.cuda.synchronize()
    for b in (0, B - 1):
        rows = sampled_rows(L, 24, 9953 + b, edge=4)
        _check_rows(q, k, v, o, lse, b, (0, 37, Hq - 1), rows, None, True, D ** -0.5,
                    f"prefill > 4 GiB, batch {b}")


def _csr_lists(B, Hq, L, seed):
    """Per query block: block 0, the diagonal block, the one before it and two random causal
    blocks; per head 48 random columns. CSR int32, sorted and unique (vectorised: 1M rows)."""
    rng = np.random.default_rng(seed)
    nqb = -(-L // 64)
    qb = np.tile(np.arange(nqb), B * Hq)
    cand = np.stack([np.zeros_like(qb), qb, np.maximum(qb - 1, 0),
                     (rng.random(qb.size) * (qb + 1)).astype(np.int64),
                     (rng.random(qb.size) * (qb + 1)).astype(np.int64)], axis=1)
    cand.sort(axis=1)
    keep = np.ones_like(cand, dtype=bool)
    keep[:, 1:] = cand[:, 1:] != cand[:, :-1]
    counts = keep.sum(axis=1)
    bptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    bidx = cand[keep].astype(np.int32)
    cols = [np.unique(rng.integers(0, L, 48)) for _ in range(B * Hq)]
    cptr = np.concatenate([[0], np.cumsum([c.size for c in cols])]).astype(np.int32)
    cidx = np.concatenate(cols).astype(np.int32)
    return bptr, bidx, cptr, cidx


def test_blocksparse_beyond_4gib():
    import torch
    import sparse_attention_attn_amd as S
    q, k, v, o, lse = _prefill_inputs()
    B, L, Hq, D = q.shape
    say(f"block-sparse B{B} L{L} Hq{Hq}: Q and O {_nbytes(q) / 1e9:.2f} GB each")
    bp, bi, cp, ci = _csr_lists(B, Hq, L, 9960)
    S.attn_blocksparse_check(bp, bi, cp, ci, B, Hq, L, L)
    dev = lambda x: torch.as_tensor(x).to(DEV)
    S.attn_fwd_blocksparse(q, k, v, o, dev(bp), dev(bi), dev(cp), dev(ci), lse=lse, causal=True,
                           scale=D ** -0.5)
    torch.cuda.synchronize()
    nqb = -(-L // 64)
    for b in (0, B - 1):
        def keys_of(h, r, b=b):
            row = (b * Hq + h) * nqb + r // 64
            return A.blocksparse_keys(bi[bp[row]:bp[row + 1]],
                                      ci[cp[b * Hq + h]:cp[b * Hq + h + 1]], L)
        rows = sampled_rows(L, 48, 9961 + b, edge=8)
        _check_rows(q, k, v, o, lse, b, (0, 37, Hq - 1), rows, keys_of, True, D ** -0.5,
                    f"block-sparse > 4 GiB, batch {b}")


def test_decode_beyond_4gib():
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, D, Lk = 16, 32, 8, 128, 131072 + 37
    q = randn_bf16_device((B, 1, Hq, D), 9970)
    k = randn_bf16_device((B, Lk, Hkv, D), 9971)
    v = randn_bf16_device((B, Lk, Hkv, D), 9972)
    assert _nbytes(k) > GIB4 and _nbytes(v) > GIB4
    say(f"decode B{B} Lk{Lk} Hkv{Hkv}: K and V {_nbytes(k) / 1e9:.2f} GB each")
    o = torch.empty((B, 1, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=DEV)
    S.attn_fwd_decode(q, k, v, o, lse, causal=True, scale=D ** -0.5)
    torch.cuda.synchronize()
    for b in (0, B - 1):
        _check_rows(q, k, v, o, lse, b, range(Hq), [0], None, True, D ** -0.5,
                    f"decode > 4 GiB, batch {b}")

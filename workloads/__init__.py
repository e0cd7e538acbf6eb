"""Seeded synthetic inputs for the attention forward path (shared by tests and bench).

This module holds NO attention arithmetic: only random-number generation, shapes and the
block-sparse index-list generator. Both the oracle side and the GPU side consume its outputs.

Recipe:
* Q/K/V: torch CPU generator seeded per tensor, float32 N(0, 1) samples rounded to bfloat16
  with round-to-nearest-even (torch's `.to(torch.bfloat16)`), contiguous [B, L, H, D].
* Workload k uses seeds 1000*k + {0: Q, 1: K, 2: V, 3: index lists, 4: sampled rows}.
* Block-sparse lists (per query head, 64x64 blocks), following the A-shape / vertical-slash /
  block-sparse pattern vocabulary of the MInference article and the per-head dynamic patterns
  of the SparseAccelerate page: key block 0 (the "first block"), the local band of the 64 key
  blocks kb in [qb-63, qb] (diagonal included), each remaining causal block kb <= qb chosen
  independently with probability 0.03, and 1000 vertical key columns drawn uniformly without
  replacement over [0, L) per head. Lists are sorted and unique.
* Vertical-slash lists (MInference article, vertical-slash pattern): per head, the slash
  offsets 0..1023 (a band of 1024 diagonals below the causal one) plus 64 offsets drawn
  uniformly from [1024, L), and 1000 vertical columns: keys 0..63 plus 936 keys drawn
  uniformly from [64, L). No key blocks.
* Structured Q/K for the dynamic index builders (`make_structured_qk`): the noise above plus a
  planted local band (a rotary code in 64 of the dims with random frequencies, so scores fall
  with the offset |i - j| like a Gaussian, to half at half a window) and planted vertical
  columns (a per-KV-head direction in the other dims, added to 1000 keys and to every query
  row). The block-sparse pipeline uses a 6144-key
  window (half height at 3072 keys, so the 96 listed blocks are about the nearest 96), a band
  rise of 6 and a column rise of 8 after the softmax scale; the vertical-slash pipeline a
  4096-key window (the rise stays above 10 over the first ~1100 offsets, the static lists'
  1024-offset band), a band rise of 12 and a column rise of 5.
* The MLA decode grid of the FlashMLA-ETAP page (section on experiments: DeepSeek-R1's 16
  heads of dimension 576, batch sizes 16 and 32, KV lengths 512 to 64K; one or two query
  tokens per the problem statement) uses the MLA recipe above with bottom-right causal
  masking. Parity cases draw it on the host like every other workload. The timing sweep
  draws it on the device (`randn_bf16_device`: a seeded device generator, same distribution
  and rounding), because the largest points hold several GB.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "randn_bf16",
    "make_qkv",
    "make_blocksparse_lists",
    "ETAP_GRID",
    "randn_bf16_device",
    "sampled_rows",
    "dense_causal_lists",
    "make_vslash_lists",
    "make_structured_qk",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # seed base = 1000 * index
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    Dqk: int
    Dv: int
    causal: bool
    scale: float
    kind: str           # "prefill" | "decode" | "mla_decode" | "blocksparse" | "vslash"
    mla: bool = False   # V is the first Dv columns of K (no separate V tensor)


WORKLOADS = {
    "tiny_causal": Workload("tiny_causal", 1, B=1, Hq=2, Hkv=2, Lq=256, Lk=256, Dqk=64, Dv=64,
                            causal=True, scale=1.0 / math.sqrt(64), kind="prefill"),
    "gqa_prefill_8k": Workload("gqa_prefill_8k", 2, B=1, Hq=32, Hkv=8, Lq=8192, Lk=8192, Dqk=128,
                               Dv=128, causal=True, scale=1.0 / math.sqrt(128), kind="prefill"),
    "gqa_decode_4k": Workload("gqa_decode_4k", 3, B=16, Hq=32, Hkv=8, Lq=1, Lk=4096, Dqk=128,
                              Dv=128, causal=False, scale=1.0 / math.sqrt(128), kind="decode"),
    "mla_decode_64k": Workload("mla_decode_64k", 4, B=8, Hq=16, Hkv=1, Lq=1, Lk=65536, Dqk=576,
                               Dv=512, causal=False, scale=1.0 / math.sqrt(192), kind="mla_decode",
                               mla=True),
    "blocksparse_128k": Workload("blocksparse_128k", 5, B=1, Hq=32, Hkv=8, Lq=131072, Lk=131072,
                                 Dqk=128, Dv=128, causal=True, scale=1.0 / math.sqrt(128),
                                 kind="blocksparse"),
    "vslash_128k": Workload("vslash_128k", 6, B=1, Hq=32, Hkv=8, Lq=131072, Lk=131072, Dqk=128,
                            Dv=128, causal=True, scale=1.0 / math.sqrt(128), kind="vslash"),
}


# FlashMLA-ETAP decode grid: (batch, query tokens, KV length) points of the MLA shape.
ETAP_GRID = {}
for _i, (_b, _lq, _lk) in enumerate((b, lq, lk) for b in (16, 32) for lq in (1, 2)
                                    for lk in (512, 1024, 2048, 4096, 8192, 16384, 32768, 65536)):
    _name = f"etap_b{_b}_q{_lq}_k{_lk}"
    ETAP_GRID[_name] = Workload(_name, 100 + _i, B=_b, Hq=16, Hkv=1, Lq=_lq, Lk=_lk, Dqk=576,
                                Dv=512, causal=True, scale=1.0 / math.sqrt(192),
                                kind="mla_decode", mla=True)
del _i, _b, _lq, _lk, _name


def randn_bf16_device(shape, seed: int, device="cuda:0") -> torch.Tensor:
    """float32 N(0,1) from a seeded generator on `device`, rounded to bf16 (RNE). For timing
    inputs only: the values differ from randn_bf16's for the same seed."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device).to(
        torch.bfloat16)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def randn_bf16(shape, seed: int) -> torch.Tensor:
    """float32 N(0,1) from a seeded CPU generator, rounded to bf16 (RNE). CPU tensor."""
    return torch.randn(tuple(shape), generator=_gen(seed), dtype=torch.float32).to(torch.bfloat16)


def make_qkv(w: Workload, b=None, lq=None, lk=None):
    """Q [B, Lq, Hq, Dqk], K [B, Lk, Hkv, Dqk], V [B, Lk, Hkv, Dv] (V is None for MLA) on CPU.

    b / lq / lk optionally override the sizes (for reduced-size parity cases of the same recipe).
    """
    B = w.B if b is None else b
    Lq = w.Lq if lq is None else lq
    Lk = w.Lk if lk is None else lk
    base = 1000 * w.index
    q = randn_bf16((B, Lq, w.Hq, w.Dqk), base + 0)
    k = randn_bf16((B, Lk, w.Hkv, w.Dqk), base + 1)
    v = None if w.mla else randn_bf16((B, Lk, w.Hkv, w.Dv), base + 2)
    return q, k, v


def make_blocksparse_lists(B, Hq, Lq, Lk, seed, block=64, local_blocks=64, p_extra=0.03,
                           n_cols=1000, first_block=True):
    """CSR index lists over (b, h, qb) -> key-block ids and over (b, h) -> key columns.

    Returns int32 numpy arrays (blk_ptr [B*Hq*nqb+1], blk_idx, col_ptr [B*Hq+1], col_idx).
    Sorted, unique, every block id < ceil(Lk/64), every column < Lk.
    The local band is aligned bottom-right: query block qb ends at query row
    min((qb+1)*64, Lq) - 1, which sees keys up to that row + Lk - Lq.
    """
    g = _gen(seed)
    nqb = -(-Lq // block)
    nkb = -(-Lk // block)
    off = Lk - Lq
    ptr = [0]
    idx_parts = []
    col_ptr = [0]
    col_parts = []
    qb_ar = np.arange(nqb)
    # last visible key block of each query block (bottom-right causal)
    last_row = np.minimum((qb_ar + 1) * block, Lq) - 1
    diag_kb = np.minimum((last_row + off) // block, nkb - 1)
    for _b in range(B):
        for _h in range(Hq):
            extra = torch.rand((nqb, nkb), generator=g).numpy() < p_extra
            kb = np.arange(nkb)[None, :]
            causal_blk = kb <= diag_kb[:, None]
            local = (kb <= diag_kb[:, None]) & (kb > diag_kb[:, None] - local_blocks)
            sel = local | (extra & causal_blk)
            if first_block:
                sel[:, 0] = True
            # row-major nonzero = per-query-block sorted key-block ids
            idx_parts.append(np.nonzero(sel)[1].astype(np.int32))
            ptr.extend((ptr[-1] + np.cumsum(sel.sum(axis=1))).tolist())
            nc = min(n_cols, Lk)
            cols = torch.randperm(Lk, generator=g)[:nc].numpy().astype(np.int32)
            cols.sort()
            col_parts.append(cols)
            col_ptr.append(col_ptr[-1] + nc)
    blk_idx = np.concatenate(idx_parts) if idx_parts else np.zeros(0, np.int32)
    col_idx = np.concatenate(col_parts) if col_parts else np.zeros(0, np.int32)
    return (np.asarray(ptr, np.int32), blk_idx.astype(np.int32),
            np.asarray(col_ptr, np.int32), col_idx.astype(np.int32))


def make_vslash_lists(B, Hq, Lk, seed, band=1024, n_far=64, n_cols=1000, sink=64):
    """Vertical-slash lists per (b, h): slash offsets (the band 0..band-1 below the diagonal plus
    n_far offsets drawn uniformly without replacement from [band, Lk)) and vertical columns
    (keys 0..sink-1 plus n_cols - sink keys drawn uniformly without replacement from
    [sink, Lk)). Returns int32 numpy arrays (slash_ptr [B*Hq+1], slash_idx, col_ptr [B*Hq+1],
    col_idx), sorted and unique."""
    g = _gen(seed)
    sp, sparts, cp, cparts = [0], [], [0], []
    for _ in range(B * Hq):
        nb = min(band, Lk)
        far = torch.randperm(max(Lk - nb, 0), generator=g)[:n_far].numpy() + nb
        offs = np.unique(np.concatenate([np.arange(nb), far])).astype(np.int32)
        sparts.append(offs)
        sp.append(sp[-1] + offs.size)
        ns = min(sink, Lk)
        rest = torch.randperm(max(Lk - ns, 0), generator=g)[:max(n_cols - ns, 0)].numpy() + ns
        cols = np.unique(np.concatenate([np.arange(ns), rest])).astype(np.int32)
        cparts.append(cols)
        cp.append(cp[-1] + cols.size)
    cat = lambda parts: np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)
    return (np.asarray(sp, np.int32), cat(sparts), np.asarray(cp, np.int32), cat(cparts))


def make_structured_qk(B, L, Hq, Hkv, D, seed, window=2048, n_cols=1000, band_logit=6.0,
                       col_logit=8.0, n_pairs=32, scale=None, device="cuda:0"):
    """Q [B, L, Hq, D] and K [B, L, Hkv, D] (bf16 on `device`) carrying the two structures the
    MInference article describes in long-context attention, planted on N(0, 1) noise: a local
    band and vertical columns. Inputs for the dynamic index builders, which find nothing in
    pure noise.

    Band: dims 0 .. 2*n_pairs-1 of every query row i and key j add a rotary code,
    a * (cos(w_m p), sin(w_m p)) at position p, for n_pairs frequencies w_m = |N(0, sigma)|
    drawn from the seeded generator with sigma = 2.355 / window. The scores then rise by
    a^2 * sum_m cos(w_m (i - j)), which averages to `band_logit` * exp(-(sigma (i - j))^2 / 2):
    the full rise at offset 0, half of it at offset window / 2, and beyond about one window
    only a random remainder of about band_logit / sqrt(2 n_pairs) (random frequencies, so no
    offset far from the diagonal is favoured twice). Columns: every KV head draws `n_cols` key positions and a unit vector u
    over the remaining dims; those keys and every query row of the group add c * u, so those
    columns' scores rise by `col_logit`. The rises are after the softmax scale (1/sqrt(D)
    unless given). Batch entries share the structure, not the noise."""
    scale = D ** -0.5 if scale is None else scale
    assert 2 * n_pairs < D
    a = math.sqrt(band_logit / (n_pairs * scale))
    c = math.sqrt(col_logit / scale)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    pos = torch.arange(L, device=device, dtype=torch.float64)
    sigma = 2.355 / window
    w = sigma * torch.randn(n_pairs, generator=g, device=device).double().abs()
    ph = pos[:, None] * w[None, :]                                      # [L, n_pairs]
    rot = torch.zeros((L, D), device=device)
    rot[:, 0:2 * n_pairs:2] = (a * torch.cos(ph)).float()
    rot[:, 1:2 * n_pairs:2] = (a * torch.sin(ph)).float()
    u = torch.zeros((Hkv, D), device=device)
    u[:, 2 * n_pairs:] = torch.randn((Hkv, D - 2 * n_pairs), generator=g, device=device)
    u = c * u / u.norm(dim=-1, keepdim=True)
    grp = Hq // Hkv
    q = torch.randn((B, L, Hq, D), generator=g, device=device)
    q += rot[None, :, None, :]
    q += u.repeat_interleave(grp, dim=0)[None, None]
    k = torch.randn((B, L, Hkv, D), generator=g, device=device)
    k += rot[None, :, None, :]
    for h in range(Hkv):
        cols = torch.randperm(L, generator=g, device=device)[:min(n_cols, L)]
        k[:, cols, h, :] += u[h]
    return q.to(torch.bfloat16), k.to(torch.bfloat16)


def dense_causal_lists(B, Hq, Lq, Lk, block=64):
    """Lists that name every causal key block and no column (block-sparse == dense causal)."""
    nqb = -(-Lq // block)
    nkb = -(-Lk // block)
    off = Lk - Lq
    ptr = [0]
    parts = []
    for _ in range(B * Hq):
        for qb in range(nqb):
            last_row = min((qb + 1) * block, Lq) - 1
            d = min((last_row + off) // block, nkb - 1)
            ids = np.arange(0, d + 1, dtype=np.int32)
            parts.append(ids)
            ptr.append(ptr[-1] + ids.size)
    return (np.asarray(ptr, np.int32), np.concatenate(parts).astype(np.int32),
            np.zeros(B * Hq + 1, np.int32), np.zeros(0, np.int32))


def sampled_rows(L, n, seed, edge=64):
    """Query rows used for sampled parity at full size: the first `edge` rows, the last `edge`
    rows, and n - 2*edge rows drawn uniformly without replacement from the rest. Sorted."""
    if n >= L:
        return np.arange(L)
    head = np.arange(0, edge)
    tail = np.arange(L - edge, L)
    mid_pool = L - 2 * edge
    m = n - 2 * edge
    mid = torch.randperm(mid_pool, generator=_gen(seed))[:m].numpy() + edge
    return np.sort(np.concatenate([head, mid, tail]))

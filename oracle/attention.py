"""Plain fp64 CPU oracle for softmax attention (dense, causal, GQA, MLA, block-sparse, split + combine).

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The product path
(the HIP library and its Python binding) never calls it, and this module imports nothing
from the product path: the two share no code, no constants and no helpers.

What it computes is the plain definition that every page reaches exactly, only faster:

* "Resumen Técnico: FlashMLA-ETAP", section "Mecanismo Central": the standard flow is
  S = Q·Kᵀ, P = softmax(S), O = P·V. The transposed flow (Sᵀ = K·Qᵀ, Pᵀ = softmax(Sᵀ),
  O = (Vᵀ·Pᵀ)ᵀ) gives the same O; `attention_transposed` evaluates that second form and
  serves only as a cross-check of this one.
* "Activar Flash Attention con llama.cpp para optimizar la inferencia", section
  "¿Qué es Flash Attention y por qué es crucial para llama.cpp?": tiling and iterative local
  updates are an implementation technique, not a change of the result. The oracle therefore
  materialises the full score matrix and applies the softmax in one go (no tiling, no online
  softmax, no reordering beyond what numpy's matmul does inside one product).
* Same page, FAQ entry on Grouped Query Attention: K and V are shared across groups of query
  heads. Reading taken: contiguous groups, KV head = query head // (Hq // Hkv).
* "Resumen Técnico: FlashMLA-ETAP", sections "Planteamiento del Problema", "Detalles de
  Implementación" and "Limitaciones Notadas por los Autores": MLA decode, 16 heads per GPU,
  head dim 576, one shared jointly-compressed latent KV, one query token per forward pass.
  Reading taken: Dqk = 576, V = the first 512 columns of the latent K, one KV head.
  `mla_value_view` builds that V as an explicit copy.
* MInference (7minutos.es article), paragraphs on the A-shape / vertical-slash /
  block-sparse patterns and on dynamically built sparse indices and masks, and
  "SparseAccelerate: Acelerando Modelos de Lenguaje", section "Patrones de Atención Dispersa
  Dinámicos": per-head sparse patterns. Reading taken: per query head, a list of 64x64 key
  blocks per 64-row query block plus a list of vertical key columns; the visible set is the
  union of both, intersected with the causal mask, each key counted once. The vertical-slash
  pattern adds per-head slash lines: diagonals at listed offsets below the causal diagonal,
  joined to the same union (`slash_row_mask`).

Readings where the pages are silent (each listed again with its reason in the design notes):
causal alignment is bottom-right (query i sees key j iff j <= i + Lk - Lq); the log-sum-exp is
the natural log of the row sum of exp(scaled, masked scores), a row with no visible key has
O = 0 and LSE = -inf; the split-KV chunk width is 64 * ceil(ceil(Lk / S) / 64).

Parity pins for every function here live in tests/test_oracle_pins.py (brute force, closed
forms, invariants, reductions to textbook cases, hand-derived golden values).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "attention",
    "attention_rows",
    "attention_query_rows",
    "attention_transposed",
    "blocksparse_row_mask",
    "combine_lse",
    "split_bounds",
    "splitkv_partials",
    "attention_splitkv",
    "mla_value_view",
    "kv_head_of",
]

# Row-sum invariant checked on every softmax the oracle forms.
_ROWSUM_TOL = 1e-12


# ---------------------------------------------------------------------------------------------
# Small named steps. Each one is a single line of the definition; the tests swap single steps
# for deliberately wrong versions to show that the pins catch such mistakes.
# ---------------------------------------------------------------------------------------------

def kv_head_of(h: int, hq: int, hkv: int) -> int:
    """GQA head map (llama.cpp page, FAQ entry on GQA): contiguous groups of g = Hq/Hkv."""
    return h // (hq // hkv)


def _scores(q_rows: np.ndarray, k_rows: np.ndarray, scale: float) -> np.ndarray:
    """S = scale · Q · Kᵀ  (FlashMLA-ETAP page, "Mecanismo Central", standard flow)."""
    return scale * (q_rows @ k_rows.T)


def _causal_visible(rows: np.ndarray, lq: int, lk: int) -> np.ndarray:
    """Bottom-right causal mask: query i sees key j iff j <= i + Lk - Lq. Shape [len(rows), Lk]."""
    j = np.arange(lk)[None, :]
    return j <= (rows[:, None] + (lk - lq))


def _softmax_rows(s: np.ndarray):
    """Row softmax over the key axis with -inf for invisible keys.

    Returns (P normalised, row max m, row sum l of exp(S - m)). Rows with no visible key give
    P = 0, m = -inf, l = 0.
    """
    m = s.max(axis=1)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    e = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for masked keys
    e[~finite, :] = 0.0
    l = e.sum(axis=1)
    p = np.zeros_like(e)
    p[finite] = e[finite] / l[finite, None]
    if finite.any():
        rs = p[finite].sum(axis=1)
        if np.max(np.abs(rs - 1.0)) > _ROWSUM_TOL:
            raise AssertionError("softmax row-sum invariant violated")
    return p, m, l


def _lse(m: np.ndarray, l: np.ndarray) -> np.ndarray:
    """LSE = m + ln l (natural log); -inf where the row has no visible key."""
    out = np.full(m.shape, -np.inf)
    ok = np.isfinite(m)
    out[ok] = m[ok] + np.log(l[ok])
    return out


def _weighted_values(p: np.ndarray, v_rows: np.ndarray) -> np.ndarray:
    """O = P · V (FlashMLA-ETAP page, "Mecanismo Central", standard flow)."""
    return p @ v_rows


# ---------------------------------------------------------------------------------------------
# Public oracle functions
# ---------------------------------------------------------------------------------------------

def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, L, H, D]")
    b, lq, hq, dqk = q.shape
    bk, lk, hkv, dk = k.shape
    bv, lv, hv, dv = v.shape
    if not (b == bk == bv and lk == lv and hkv == hv and dqk == dk):
        raise ValueError("inconsistent q/k/v shapes")
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return b, lq, hq, dqk, lk, hkv, dv


def attention_rows(q, k, v, scale, causal, b, h, rows, allowed=None):
    """Attention output for a subset of query rows of one (batch, query head).

    q: [B, Lq, Hq, Dqk], k: [B, Lk, Hkv, Dqk], v: [B, Lk, Hkv, Dv] (any float dtype; computed in
    fp64). rows: 1-D int array of query positions. allowed: None or a bool array
    [len(rows), Lk] of extra visibility (block-sparse union), ANDed with the causal mask.
    Returns (O [len(rows), Dv] fp64, LSE [len(rows)] fp64).
    """
    _, lq, hq, _, _, _, _ = _check_shapes(q, k, v)
    rows = np.asarray(rows, dtype=np.int64)
    return attention_query_rows(q[b, rows, h, :], k, v, scale, causal, b, h, rows, lq, hq, allowed)


def attention_query_rows(q_rows, k, v, scale, causal, b, h, rows, lq, hq, allowed=None):
    """As `attention_rows`, with the query rows given directly: q_rows [len(rows), Dqk] holds
    Q[b, rows, h, :] of a query tensor with Lq = lq positions and Hq = hq heads."""
    lk, hkv = k.shape[1], k.shape[2]
    rows = np.asarray(rows, dtype=np.int64)
    kvh = kv_head_of(h, hq, hkv)
    qr = np.asarray(q_rows, dtype=np.float64)
    kr = np.asarray(k[b, :, kvh, :], dtype=np.float64)
    vr = np.asarray(v[b, :, kvh, :], dtype=np.float64)
    s = _scores(qr, kr, np.float64(scale))
    visible = np.ones(s.shape, dtype=bool)
    if causal:
        visible &= _causal_visible(rows, lq, lk)
    if allowed is not None:
        visible &= allowed
    s = np.where(visible, s, -np.inf)
    p, m, l = _softmax_rows(s)
    return _weighted_values(p, vr), _lse(m, l)


def attention(q, k, v, scale, causal, allowed_fn=None, row_chunk=4096):
    """Full attention. Returns (O [B, Lq, Hq, Dv], LSE [B, Hq, Lq]) in fp64.

    allowed_fn: None, or a callable (b, h, rows) -> bool [len(rows), Lk] giving the sparse
    visibility of those rows (see `blocksparse_row_mask`).
    """
    bsz, lq, hq, _, lk, hkv, dv = _check_shapes(q, k, v)
    o = np.zeros((bsz, lq, hq, dv))
    lse = np.zeros((bsz, hq, lq))
    for b in range(bsz):
        for h in range(hq):
            for r0 in range(0, lq, row_chunk):
                rows = np.arange(r0, min(lq, r0 + row_chunk))
                allowed = None if allowed_fn is None else allowed_fn(b, h, rows)
                orow, lrow = attention_rows(q, k, v, scale, causal, b, h, rows, allowed)
                o[b, rows, h, :] = orow
                lse[b, h, rows] = lrow
    return o, lse


def attention_transposed(q, k, v, scale, causal):
    """The transposed flow of the FlashMLA-ETAP page ("Mecanismo Central"), in fp64.

    Sᵀ = K·Qᵀ (keys × queries), Pᵀ = softmax over the key axis (axis 0), O = (Vᵀ·Pᵀ)ᵀ.
    Written independently of `attention` as a second formulation to cross-check it.
    """
    bsz, lq, hq, _, lk, hkv, dv = _check_shapes(q, k, v)
    g = hq // hkv
    o = np.zeros((bsz, lq, hq, dv))
    for b in range(bsz):
        for h in range(hq):
            kk = np.asarray(k[b, :, h // g, :], np.float64)
            vv = np.asarray(v[b, :, h // g, :], np.float64)
            qq = np.asarray(q[b, :, h, :], np.float64)
            st = np.float64(scale) * (kk @ qq.T)                      # [Lk, Lq]
            if causal:
                i = np.arange(lq)[None, :]
                j = np.arange(lk)[:, None]
                st = np.where(j <= i + (lk - lq), st, -np.inf)
            col_max = st.max(axis=0)
            safe = np.where(np.isfinite(col_max), col_max, 0.0)
            et = np.exp(st - safe[None, :])
            den = et.sum(axis=0)
            pt = np.divide(et, den[None, :], out=np.zeros_like(et), where=den[None, :] > 0)
            o[b, :, h, :] = (vv.T @ pt).T
    return o


def mla_value_view(k_latent: np.ndarray, dv: int = 512) -> np.ndarray:
    """MLA value tensor: an explicit copy of the first `dv` latent columns of K.

    (FlashMLA-ETAP page, "Detalles de Implementación": one jointly low-rank-compressed latent
    KV. Reading: V = K[..., :512] of the 576-wide latent, 576 = 512 latent + 64 rope.)
    """
    return np.array(k_latent[..., :dv], dtype=np.float64, copy=True)


# ---------------------------------------------------------------------------------------------
# Block-sparse visibility from CSR index lists
# ---------------------------------------------------------------------------------------------

def blocksparse_row_mask(rows, lk, blocks_of_qb, cols, block_m=64, block_n=64):
    """Visible-key mask [len(rows), Lk] of the block/column union for one (batch, query head).

    blocks_of_qb: callable qb -> 1-D int array of key-block ids listed for query block qb.
    cols: 1-D int array of vertical key columns of this head.
    allowed(i, j) = (j // block_n in blocks[i // block_m]) or (j in cols). Causality is applied
    separately by the caller, on top. Built with np.repeat of a per-block bitmap and a column
    bitmap: deliberately a different construction from any gather / de-duplication walk.
    """
    rows = np.asarray(rows, dtype=np.int64)
    nkb = (lk + block_n - 1) // block_n
    colmask = np.zeros(lk, dtype=bool)
    cols = np.asarray(cols, dtype=np.int64)
    if cols.size:
        colmask[cols] = True
    out = np.zeros((rows.size, lk), dtype=bool)
    for qb in np.unique(rows // block_m):
        bm = np.zeros(nkb, dtype=bool)
        blk = np.asarray(blocks_of_qb(int(qb)), dtype=np.int64)
        if blk.size:
            bm[blk] = True
        keymask = np.repeat(bm, block_n)[:lk] | colmask
        out[(rows // block_m) == qb] = keymask
    return out


def csr_allowed_fn(blk_ptr, blk_idx, col_ptr, col_idx, hq, nqb, lk, block_m=64, block_n=64):
    """Adapter: CSR lists (as laid out at the library boundary) -> allowed_fn for `attention`.

    blk_ptr has B*Hq*nqb + 1 entries over (b, h, qb) row-major; col_ptr has B*Hq + 1 over (b, h).
    """
    blk_ptr = np.asarray(blk_ptr, np.int64)
    blk_idx = np.asarray(blk_idx, np.int64)
    col_ptr = np.asarray(col_ptr, np.int64)
    col_idx = np.asarray(col_idx, np.int64)

    def fn(b, h, rows):
        base = (b * hq + h) * nqb

        def blocks_of_qb(qb):
            r = base + qb
            return blk_idx[blk_ptr[r]:blk_ptr[r + 1]]

        c = (b * hq + h)
        return blocksparse_row_mask(rows, lk, blocks_of_qb, col_idx[col_ptr[c]:col_ptr[c + 1]],
                                    block_m, block_n)

    return fn


def blocksparse_keys(blocks, cols, lk, block_n=64):
    """Sorted key positions of the block/column union for one query block: every key of the
    listed blocks and every listed column, each once, inside [0, Lk)."""
    parts = [np.arange(int(kb) * block_n, min((int(kb) + 1) * block_n, lk), dtype=np.int64)
             for kb in np.asarray(blocks, dtype=np.int64)]
    parts.append(np.asarray(cols, dtype=np.int64))
    keys = np.unique(np.concatenate(parts)) if parts else np.zeros(0, np.int64)
    return keys[(keys >= 0) & (keys < lk)]


def attention_rows_over_keys(q_rows, rows, k_head, v_head, scale, keys, lq, lk, causal):
    """Attention of some query rows of one (batch, query head) when only `keys` can be visible:
    the plain definition with the score matrix restricted to those columns (the other keys
    have weight zero by the mask), the causal limit applied per row.

    q_rows [n, Dqk]; k_head [Lk, Dqk]; v_head [Lk, Dv]; keys sorted. Returns (O [n, Dv], LSE [n]).
    """
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    s = _scores(np.asarray(q_rows, np.float64), np.asarray(k_head, np.float64)[keys],
                np.float64(scale))
    if causal:
        s = np.where(keys[None, :] <= (rows + lk - lq)[:, None], s, -np.inf)
    p, m, l = _softmax_rows(s)
    return _weighted_values(p, np.asarray(v_head, np.float64)[keys]), _lse(m, l)


def slash_row_mask(rows, lq, lk, offsets):
    """Visible-key mask [len(rows), Lk] of the slash lines of one (batch, query head).

    A slash line at offset o >= 0 is the diagonal o keys below the causal one: query row i sees
    key i + (Lk - Lq) - o when that key exists (MInference article, paragraph on the
    vertical-slash pattern; reading: the diagonal is bottom-right aligned like the causal mask,
    offsets are counted downward from it). Built by scattering each listed diagonal into the
    mask, one offset at a time.
    """
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, lk), dtype=bool)
    for o in np.asarray(offsets, dtype=np.int64):
        keys = rows + (lk - lq) - o
        ok = (o >= 0) & (keys >= 0) & (keys < lk)
        out[np.nonzero(ok)[0], keys[ok]] = True
    return out


def vslash_allowed_fn(blk_ptr, blk_idx, col_ptr, col_idx, sl_ptr, sl_idx, hq, nqb, lq, lk,
                      block_m=64, block_n=64):
    """Adapter like `csr_allowed_fn`, with per-head slash offsets added to the union:
    sl_ptr has B*Hq + 1 entries over (b, h); sl_idx holds the offsets."""
    blocks_cols = csr_allowed_fn(blk_ptr, blk_idx, col_ptr, col_idx, hq, nqb, lk, block_m,
                                 block_n)
    sl_ptr = np.asarray(sl_ptr, np.int64)
    sl_idx = np.asarray(sl_idx, np.int64)

    def fn(b, h, rows):
        c = b * hq + h
        return blocks_cols(b, h, rows) | slash_row_mask(rows, lq, lk,
                                                        sl_idx[sl_ptr[c]:sl_ptr[c + 1]])

    return fn


# ---------------------------------------------------------------------------------------------
# Split-KV partials and their log-sum-exp combine
# ---------------------------------------------------------------------------------------------

def split_bounds(lk: int, num_splits: int):
    """Key ranges [lo, hi) of each split: chunk width C = 64 * ceil(ceil(Lk / S) / 64).

    Trailing splits may be empty (lo >= hi); they contribute weight 0.
    """
    per = -(-lk // num_splits)
    c = 64 * (-(-per // 64))
    return [(min(s * c, lk), min((s + 1) * c, lk)) for s in range(num_splits)]


def splitkv_partials(q, k, v, scale, causal, num_splits):
    """Per-split normalised partial outputs and LSEs.

    Returns (O_part [S, B, Hq, Lq, Dv], LSE_part [S, B, Hq, Lq]) in fp64. Split s attends only to
    keys in its range (and the causal mask); an empty visible set gives O_s = 0, LSE_s = -inf.
    """
    bsz, lq, hq, _, lk, hkv, dv = _check_shapes(q, k, v)
    bounds = split_bounds(lk, num_splits)
    o_part = np.zeros((num_splits, bsz, hq, lq, dv))
    lse_part = np.full((num_splits, bsz, hq, lq), -np.inf)
    rows = np.arange(lq)
    for s, (lo, hi) in enumerate(bounds):
        inrange = np.zeros((lq, lk), dtype=bool)
        inrange[:, lo:hi] = True
        for b in range(bsz):
            for h in range(hq):
                orow, lrow = attention_rows(q, k, v, scale, causal, b, h, rows, inrange)
                o_part[s, b, h] = orow
                lse_part[s, b, h] = lrow
    return o_part, lse_part


def combine_lse(o_part, lse_part):
    """Merge split partials: M = max_s LSE_s, w_s = exp(LSE_s - M), LSE = M + ln Σ w_s,
    O = Σ w_s O_s / Σ w_s. If every split is empty: O = 0, LSE = -inf.

    o_part: [S, ..., Dv], lse_part: [S, ...]. Returns (O [..., Dv], LSE [...]) in fp64.
    """
    o_part = np.asarray(o_part, np.float64)
    lse_part = np.asarray(lse_part, np.float64)
    mx = lse_part.max(axis=0)
    ok = np.isfinite(mx)
    safe = np.where(ok, mx, 0.0)
    w = np.exp(lse_part - safe[None])              # exp(-inf) = 0
    w = np.where(ok[None], w, 0.0)
    den = w.sum(axis=0)
    num = (w[..., None] * o_part).sum(axis=0)
    o = np.zeros(num.shape)
    o[ok] = num[ok] / den[ok][..., None]
    lse = np.full(mx.shape, -np.inf)
    lse[ok] = mx[ok] + np.log(den[ok])
    return o, lse


def attention_splitkv(q, k, v, scale, causal, num_splits):
    """Split-KV attention: partials per split, then the LSE combine. Returns (O, LSE[B,Hq,Lq])."""
    o_part, lse_part = splitkv_partials(q, k, v, scale, causal, num_splits)
    o, lse = combine_lse(o_part, lse_part)        # o: [B, Hq, Lq, Dv]
    return np.transpose(o, (0, 2, 1, 3)), lse


def effective_scale(scale) -> float:
    """The fp32 value the GPU receives, as fp64 (scale crosses the boundary as a C float)."""
    return float(np.float32(scale))

"""Plain fp64 CPU oracle for the dynamic sparse-index builder (block and column lists from Q, K).

TEST INFRASTRUCTURE ONLY. Only the test suite may import or call this module. The product path
(the HIP library and its Python binding) never calls it, and this module imports nothing from
the product path.

What the pages fix and what they leave open:

* MInference (7minutos.es article), paragraphs on the three patterns and on dynamic sparse
  indices: attention weights in long contexts are sparse and input-dependent; each head follows
  a pattern (A-shape, vertical-slash, block-sparse); the sparse indices are built on the fly
  during inference with a fast approximation, per head. The same article notes that a small
  set of top columns carries most of the attention mass.
* "SparseAccelerate: Acelerando Modelos de Lenguaje", section "Patrones de Atención Dispersa
  Dinámicos": per-head dynamic patterns chosen for the input.

The pages name no estimator. The one computed here is a reading of them, the plainest that
the lists consumed by the block-sparse forward admit:

1. Block lists (per query head, per 64-row query block qb): mean-pool the query block's rows
   and every 64-key block's rows; score each causal key block kb <= qb by scale * <mean q,
   mean k>; keep the diagonal block qb and the top (topk - 1) other causal blocks, ranked by
   score, ties to the lower block id. A query block therefore lists min(topk, qb + 1) blocks.
2. Column lists (per query head): probe with the last `probe` query rows; each probe row's
   softmax over its causally visible keys; a key's importance is the sum of its probability
   over the probe rows; keep the top n_cols keys, ties to the lower key index.
3. Slash lists (per query head, for the vertical-slash pattern): the same probe; the slash
   line at offset o is the diagonal o keys below the causal one (probe row r meets key r - o);
   its importance is the sum over probe rows of their probability on that key; keep the top
   n_slash offsets, ties to the lower offset.

Sizes are square and causal (Lq = Lk = L). Lists are sorted ascending, as the consumer needs.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "pooled_rows",
    "block_scores",
    "select_blocks",
    "probe_importance",
    "select_columns",
    "build_index",
    "block_count",
    "slash_importance",
    "build_vslash_index",
]


def pooled_rows(x: np.ndarray, block: int) -> np.ndarray:
    """Mean of each group of `block` consecutive rows of x [L, D]; the last group averages the
    rows it has."""
    L = x.shape[0]
    n = -(-L // block)
    out = np.empty((n, x.shape[1]), dtype=np.float64)
    for i in range(n):
        out[i] = x[i * block:min((i + 1) * block, L)].mean(axis=0)
    return out


def block_scores(q_head: np.ndarray, k_head: np.ndarray, scale: float, block: int) -> np.ndarray:
    """scale * pooled(q) @ pooled(k)^T, [nqb, nkb], with -inf above the causal diagonal."""
    s = scale * (pooled_rows(q_head, block) @ pooled_rows(k_head, block).T)
    nqb, nkb = s.shape
    s[np.arange(nkb)[None, :] > np.arange(nqb)[:, None]] = -np.inf
    return s


def block_count(qb: int, topk: int) -> int:
    """Blocks listed for query block qb."""
    return min(topk, qb + 1)


def select_blocks(scores_row: np.ndarray, qb: int, topk: int) -> np.ndarray:
    """The diagonal block plus the top (topk - 1) other causal blocks of one query block, ties to
    the lower block id; sorted ascending."""
    others = [kb for kb in range(qb)]
    others.sort(key=lambda kb: (-scores_row[kb], kb))
    chosen = sorted(others[:max(0, topk - 1)] + [qb])
    return np.asarray(chosen, dtype=np.int32)


def probe_importance(q_head: np.ndarray, k_head: np.ndarray, scale: float, probe: int) -> np.ndarray:
    """Sum over the last `probe` query rows of their causal softmax probabilities, per key."""
    L = q_head.shape[0]
    rows = np.arange(max(0, L - probe), L)
    s = scale * (q_head[rows] @ k_head.T)                  # [P, L]
    s[np.arange(L)[None, :] > rows[:, None]] = -np.inf     # row r sees keys j <= r
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p /= p.sum(axis=1, keepdims=True)
    return p.sum(axis=0)


def slash_importance(q_head: np.ndarray, k_head: np.ndarray, scale: float, probe: int) -> np.ndarray:
    """Per diagonal offset o in [0, L): the sum over the last `probe` query rows r of their
    causal softmax probability on key r - o (rows with r < o do not meet that line)."""
    L = q_head.shape[0]
    rows = np.arange(max(0, L - probe), L)
    s = scale * (q_head[rows] @ k_head.T)
    s[np.arange(L)[None, :] > rows[:, None]] = -np.inf
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p /= p.sum(axis=1, keepdims=True)
    imp = np.zeros(L)
    for a, r in enumerate(rows):
        imp[:r + 1] += p[a, r::-1]     # offsets 0..r meet keys r, r-1, ..., 0
    return imp


def select_columns(importance: np.ndarray, n_cols: int) -> np.ndarray:
    """The n_cols keys of largest importance, ties to the lower index; sorted ascending."""
    order = sorted(range(importance.shape[0]), key=lambda j: (-importance[j], j))
    return np.asarray(sorted(order[:min(n_cols, importance.shape[0])]), dtype=np.int32)


def build_index(q, k, scale, topk, n_cols, block=64, probe=64):
    """CSR lists for q [B, L, Hq, D], k [B, L, Hkv, D] (fp64 arrays, contiguous KV-head groups):
    blk_ptr [B*Hq*nqb + 1], blk_idx, col_ptr [B*Hq + 1], col_idx (int32 numpy arrays).

    Also returns, for validity checks, the block scores [B, Hq, nqb, nkb] and the column
    importances [B, Hq, L]."""
    B, L, Hq, _ = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    nqb = -(-L // block)
    blk_ptr, blk_parts, col_ptr, col_parts = [0], [], [0], []
    scores_all = np.empty((B, Hq, nqb, nqb))
    imp_all = np.empty((B, Hq, L))
    for b in range(B):
        for h in range(Hq):
            qh = q[b, :, h, :]
            kh = k[b, :, h // g, :]
            sc = block_scores(qh, kh, scale, block)
            scores_all[b, h] = sc
            for qb in range(nqb):
                ids = select_blocks(sc[qb], qb, topk)
                blk_parts.append(ids)
                blk_ptr.append(blk_ptr[-1] + ids.size)
            imp = probe_importance(qh, kh, scale, probe)
            imp_all[b, h] = imp
            cols = select_columns(imp, n_cols)
            col_parts.append(cols)
            col_ptr.append(col_ptr[-1] + cols.size)
    cat = lambda parts: (np.concatenate(parts) if parts else np.zeros(0)).astype(np.int32)
    return (np.asarray(blk_ptr, np.int32), cat(blk_parts), np.asarray(col_ptr, np.int32),
            cat(col_parts), scores_all, imp_all)


def build_vslash_index(q, k, scale, n_cols, n_slash, probe=64):
    """Vertical-slash lists for q [B, L, Hq, D], k [B, L, Hkv, D] (fp64 arrays): col_ptr
    [B*Hq + 1], col_idx, slash_ptr [B*Hq + 1], slash_idx (int32), plus the column and slash
    importances [B, Hq, L] for validity checks. Columns as in `build_index`; offsets are the
    top n_slash of `slash_importance` (ties to the lower offset), sorted ascending."""
    B, L, Hq, _ = q.shape
    g = Hq // k.shape[2]
    col_ptr, col_parts, sl_ptr, sl_parts = [0], [], [0], []
    cimp = np.empty((B, Hq, L))
    simp = np.empty((B, Hq, L))
    for b in range(B):
        for h in range(Hq):
            qh = q[b, :, h, :]
            kh = k[b, :, h // g, :]
            cimp[b, h] = probe_importance(qh, kh, scale, probe)
            simp[b, h] = slash_importance(qh, kh, scale, probe)
            cols = select_columns(cimp[b, h], n_cols)
            offs = select_columns(simp[b, h], n_slash)   # same ranking rule over offsets
            col_parts.append(cols)
            col_ptr.append(col_ptr[-1] + cols.size)
            sl_parts.append(offs)
            sl_ptr.append(sl_ptr[-1] + offs.size)
    cat = lambda parts: (np.concatenate(parts) if parts else np.zeros(0)).astype(np.int32)
    return (np.asarray(col_ptr, np.int32), cat(col_parts), np.asarray(sl_ptr, np.int32),
            cat(sl_parts), cimp, simp)

"""CPU check that the near-tie band of the index-builder parity tests stays narrow at the
128K workloads' shape (B 1, Hq 32, Hkv 8, L 131072, D 128).

The GPU tests accept a column or slash line the oracle did not pick only when its oracle score
lies within TOPK_REL_TOL of the k-th value. This computes, with the oracle, which oracle ranks
that band reaches for the heads the full-size GPU tests check, so a wider tolerance cannot slip
in unnoticed: each band must stay within a few ranks of k."""

import numpy as np
import pytest

from oracle import sparse_index as X
from tests.helpers import TOPK_RANK_SLACK, TOPK_REL_TOL, topk_band_ranks
from workloads import WORKLOADS, make_qkv

MAX_BAND_RANKS = 8   # ranks on either side of k that the band may reach


@pytest.mark.parametrize("name,heads,n_cols,n_slash", [
    ("blocksparse_128k", (0, 29), 1000, 0),
    ("vslash_128k", (3, 30), 1000, 1088),
])
def test_band_rank_width_at_128k(name, heads, n_cols, n_slash):
    w = WORKLOADS[name]
    q, k, _ = make_qkv(w)
    sc = float(np.float32(w.scale))
    g = w.Hq // w.Hkv
    assert MAX_BAND_RANKS <= TOPK_RANK_SLACK
    for h in heads:
        qh = q[0, :, h].double().numpy()
        kh = k[0, :, h // g].double().numpy()
        checks = [("columns", X.probe_importance(qh, kh, sc, 64), n_cols)]
        if n_slash:
            checks.append(("slash lines", X.slash_importance(qh, kh, sc, 64), n_slash))
        for what, imp, kk in checks:
            lo, hi = topk_band_ranks(imp, kk, TOPK_REL_TOL)
            print(f"{name} head {h} {what}: band reaches ranks {lo}..{hi} around {kk}")
            assert kk - lo <= MAX_BAND_RANKS and hi - kk <= MAX_BAND_RANKS, (
                f"{name} head {h} {what}: the near-tie band reaches ranks {lo}..{hi} around {kk}")


def test_band_helper_counts_ranks():
    """topk_band_ranks on a hand-made list: scores 10, 9, ..., 1; k = 5 (score 6); a relative
    band of 0.2 (1.2) reaches scores 7.2 down to 4.8, i.e. ranks 4..6."""
    scores = np.arange(10, 0, -1, dtype=np.float64)
    assert topk_band_ranks(scores, 5, 0.2) == (4, 6)
    assert topk_band_ranks(scores, 5, 0.0) == (5, 5)

"""Shared test utilities: tolerance checks of GPU results against the fp64 oracle."""

from __future__ import annotations

import json
import os
import sys

import numpy as np

# Parity bar: bf16 inputs, fp32 accumulation. O within max-abs 1e-2 and mean-abs 1e-3 of the
# fp64 oracle, LSE (natural log) within max-abs 1e-3.
O_MAX_ABS = 1e-2
O_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3


# Top-k lists decided in fp32 on the GPU and in fp64 by the oracle may differ only at near-ties.
# Column and slash-line importances are positive sums of probabilities whose fp32 error is about
# 1e-5 of their value, so a swapped id must score within TOPK_REL_TOL of the k-th value
# (relative); block scores sit near zero, so theirs is relative to 1 + |k-th|. Every swapped
# id must also sit within TOPK_RANK_SLACK places of the k-th in the oracle's ranking.
TOPK_REL_TOL = 1e-4
TOPK_BLOCK_TOL = 2e-4
TOPK_RANK_SLACK = 16


def topk_band_ranks(scores, k, rel_tol=TOPK_REL_TOL):
    """1-based range of oracle ranks whose score lies within rel_tol·|k-th| of the k-th largest
    score: the ranks a near-tie swap under that band can reach."""
    srt = np.sort(np.asarray(scores, np.float64))[::-1]
    kth = srt[k - 1]
    band = rel_tol * abs(kth)
    return int(np.sum(srt > kth + band)) + 1, int(np.sum(srt >= kth - band))


def say(msg: str):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_f64(t) -> np.ndarray:
    """bf16/fp32 torch tensor (any device) -> fp64 numpy (exact widening)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def lse_diff(a, b) -> np.ndarray:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(same_inf, 0.0, np.abs(a - b))
    d[np.isnan(d)] = np.inf
    return d


def check_parity(o_gpu, o_ref, lse_gpu=None, lse_ref=None, label="", record=None):
    """Element-by-element comparison; returns a stats dict, asserts the parity bar.

    record: a workload name. When the environment variable ATTN_PARITY_LOG names a file, the
    stats (with the sums needed to merge several calls of one workload) are appended to it as
    one JSON line, for tests/parity_table.py."""
    o_gpu = np.asarray(o_gpu, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{label}: non-finite O"
    d = np.abs(o_gpu - o_ref)
    ref_sq = float(np.sum(o_ref * o_ref))
    stats = {
        "o_max_abs": float(d.max(initial=0.0)),
        "o_mean_abs": float(d.mean()) if d.size else 0.0,
        "o_rmse": float(np.sqrt(np.mean(d * d))) if d.size else 0.0,
        "o_rel_rmse": float(np.sqrt(np.sum(d * d) / ref_sq)) if ref_sq > 0 else 0.0,
    }
    worst = np.unravel_index(int(np.argmax(d)), d.shape) if d.size else None
    if lse_gpu is not None:
        dl = lse_diff(lse_gpu, lse_ref)
        stats["lse_max_abs"] = float(dl.max(initial=0.0))
    print(f"[parity] {label} {stats}", flush=True)
    log = os.environ.get("ATTN_PARITY_LOG")
    if record and log:
        rec = {"workload": record, "label": label, "n": int(d.size),
               "o_sum_abs": float(d.sum()), "o_sum_sq": float(np.sum(d * d)),
               "o_ref_sum_sq": ref_sq, **stats}
        with open(log, "a") as f:
            f.write(json.dumps(rec) + "\n")
    assert stats["o_max_abs"] <= O_MAX_ABS, f"{label}: O max-abs {stats['o_max_abs']} at {worst} " \
        f"(gpu {o_gpu[worst]}, ref {o_ref[worst]})"
    assert stats["o_mean_abs"] <= O_MEAN_ABS, f"{label}: O mean-abs {stats['o_mean_abs']}"
    if lse_gpu is not None:
        assert stats["lse_max_abs"] <= LSE_MAX_ABS, f"{label}: LSE max-abs {stats['lse_max_abs']}"
    return stats

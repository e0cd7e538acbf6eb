"""Shared test utilities: tolerance checks of GPU results against the fp64 oracle."""

from __future__ import annotations

import sys

import numpy as np

# Parity bar: bf16 inputs, fp32 accumulation. O within max-abs 1e-2 and mean-abs 1e-3 of the
# fp64 oracle, LSE (natural log) within max-abs 1e-3.
O_MAX_ABS = 1e-2
O_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3


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


def check_parity(o_gpu, o_ref, lse_gpu=None, lse_ref=None, label=""):
    """Element-by-element comparison; returns a stats dict, asserts the parity bar."""
    o_gpu = np.asarray(o_gpu, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{label}: non-finite O"
    d = np.abs(o_gpu - o_ref)
    stats = {
        "o_max_abs": float(d.max(initial=0.0)),
        "o_mean_abs": float(d.mean()) if d.size else 0.0,
        "o_rmse": float(np.sqrt(np.mean(d * d))) if d.size else 0.0,
    }
    worst = np.unravel_index(int(np.argmax(d)), d.shape) if d.size else None
    if lse_gpu is not None:
        dl = lse_diff(lse_gpu, lse_ref)
        stats["lse_max_abs"] = float(dl.max(initial=0.0))
    print(f"[parity] {label} {stats}", flush=True)
    assert stats["o_max_abs"] <= O_MAX_ABS, f"{label}: O max-abs {stats['o_max_abs']} at {worst} " \
        f"(gpu {o_gpu[worst]}, ref {o_ref[worst]})"
    assert stats["o_mean_abs"] <= O_MEAN_ABS, f"{label}: O mean-abs {stats['o_mean_abs']}"
    if lse_gpu is not None:
        assert stats["lse_max_abs"] <= LSE_MAX_ABS, f"{label}: LSE max-abs {stats['lse_max_abs']}"
    return stats

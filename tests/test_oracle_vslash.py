"""Pins of the oracle's slash-line visibility (vertical-slash pattern), CPU only, and planted
mistakes that the pins must catch.

Slash line o: query row i sees key i + (Lk - Lq) - o. The pins: brute force with the definition
written as a scalar predicate; closed forms (offset 0 alone returns V on the aligned diagonal
with LSE = scale q.k; offset 0 plus column 0 is a two-key mix, and row 0 sees key 0 once);
reductions (every offset = dense causal; offsets 0..w-1 = a sliding window of width w); the
bottom-right alignment with Lq < Lk; and a slash inside a listed block adds nothing.
"""

import math

import numpy as np
import pytest

from oracle import attention as A
from oracle.bruteforce import attention_bruteforce


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _close(a, b, tol=1e-12):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    assert np.max(np.abs(a[fin] - b[fin]), initial=0.0) <= tol


def _vs(q, k, v, scale, offsets, cols=(), blocks=None, causal=True, bs=64):
    """Attention with one slash list and one column list shared by every head."""
    B, Lq, Hq, _ = q.shape
    Lk = k.shape[1]
    nqb = -(-Lq // bs)
    bp, bi = [0], []
    for _ in range(B * Hq):
        for qb in range(nqb):
            ids = sorted((blocks or {}).get(qb, []))
            bi += ids
            bp.append(len(bi))
    cp = [len(cols) * i for i in range(B * Hq + 1)]
    ci = list(cols) * (B * Hq)
    sp = [len(offsets) * i for i in range(B * Hq + 1)]
    si = list(offsets) * (B * Hq)
    fn = A.vslash_allowed_fn(bp, bi, cp, ci, sp, si, Hq, nqb, Lq, Lk, bs, bs)
    return A.attention(q, k, v, scale, causal, allowed_fn=fn)


@pytest.mark.parametrize("seed", [0, 1])
def test_bruteforce_vertical_slash(seed):
    B, Hq, Hkv, Lq, Lk, D = 1, 2, 1, 9, 13, 3
    q, k, v = _rand((B, Lq, Hq, D), seed), _rand((B, Lk, Hkv, D), seed + 5), _rand((B, Lk, Hkv, D), seed + 9)
    offs, cols = [0, 2, 7], [1, 10]
    o, lse = _vs(q, k, v, 0.8, offs, cols, bs=4)
    vis = lambda b, h, i, j: (i + (Lk - Lq) - j) in offs or j in cols
    ob, lb = attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), 0.8, True, vis)
    _close(o, ob)
    _close(lse, lb)


def test_offset_zero_alone_returns_diagonal_values():
    B, Hq, L, D, scale = 1, 2, 50, 4, 0.6
    q, k, v = _rand((B, L, Hq, D), 1), _rand((B, L, Hq, D), 2), _rand((B, L, Hq, D), 3)
    o, lse = _vs(q, k, v, scale, [0])
    _close(o, v)
    _close(lse, scale * np.einsum("blhd,blhd->bhl", q, k))


def test_alignment_is_bottom_right():
    """Lq < Lk: offset 0 pairs query i with key i + Lk - Lq."""
    B, Hq, Lq, Lk, D, scale = 1, 1, 20, 70, 4, 0.5
    q, k, v = _rand((B, Lq, Hq, D), 4), _rand((B, Lk, Hq, D), 5), _rand((B, Lk, Hq, D), 6)
    o, lse = _vs(q, k, v, scale, [0])
    _close(o, v[:, Lk - Lq:])
    _close(lse, scale * np.einsum("blhd,blhd->bhl", q, k[:, Lk - Lq:]))


def test_offset_zero_and_column_zero_two_key_mix():
    """Row 0 sees key 0 once (slash and column coincide); row i > 0 mixes keys 0 and i."""
    B, Hq, L, D, scale = 1, 1, 30, 4, 0.7
    q, k, v = _rand((B, L, Hq, D), 7), _rand((B, L, Hq, D), 8), _rand((B, L, Hq, D), 9)
    o, lse = _vs(q, k, v, scale, [0], cols=[0])
    _close(o[0, 0, 0], v[0, 0, 0])
    _close(lse[0, 0, 0], scale * q[0, 0, 0] @ k[0, 0, 0])
    for i in range(1, L):
        s0, si = scale * q[0, i, 0] @ k[0, 0, 0], scale * q[0, i, 0] @ k[0, i, 0]
        w = 1.0 / (1.0 + math.exp(s0 - si))
        _close(o[0, i, 0], w * v[0, i, 0] + (1 - w) * v[0, 0, 0], 1e-12)
        _close(lse[0, 0, i], max(s0, si) + math.log1p(math.exp(-abs(s0 - si))), 1e-12)


def test_every_offset_is_dense_causal():
    B, Hq, Hkv, L, D = 1, 4, 2, 90, 8
    q, k, v = _rand((B, L, Hq, D), 10), _rand((B, L, Hkv, D), 11), _rand((B, L, Hkv, D), 12)
    o, lse = _vs(q, k, v, 0.3, list(range(L)))
    od, ld = A.attention(q, k, v, 0.3, True)
    _close(o, od)
    _close(lse, ld)


def test_band_of_offsets_is_a_sliding_window():
    """Offsets 0..w-1: row i sees keys max(0, i - w + 1) .. i, written as its own prefix sums."""
    B, Hq, L, D, w, scale = 1, 1, 40, 3, 6, 0.9
    q, k, v = _rand((B, L, Hq, D), 13), _rand((B, L, Hq, D), 14), _rand((B, L, Hq, D), 15)
    o, lse = _vs(q, k, v, scale, list(range(w)))
    for i in range(L):
        js = range(max(0, i - w + 1), i + 1)
        s = [scale * float(q[0, i, 0] @ k[0, j, 0]) for j in js]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        tot = math.fsum(e)
        ref = sum(ei * v[0, j, 0] for ei, j in zip(e, js)) / tot
        _close(o[0, i, 0], ref, 1e-12)
        _close(lse[0, 0, i], mx + math.log(tot), 1e-12)


def test_slash_inside_listed_block_adds_nothing():
    B, Hq, L, D = 1, 1, 128, 4
    q, k, v = _rand((B, L, Hq, D), 16), _rand((B, L, Hq, D), 17), _rand((B, L, Hq, D), 18)
    blocks = {0: [0], 1: [0, 1]}   # every slash key of these rows lies in a listed block
    o1, l1 = _vs(q, k, v, 0.5, [], blocks=blocks)
    o2, l2 = _vs(q, k, v, 0.5, [0, 3, 63], blocks=blocks)
    _close(o1, o2)
    _close(l1, l2)


# ---- planted mistakes ---------------------------------------------------------------------
def _pins():
    return [lambda: test_bruteforce_vertical_slash(0), test_offset_zero_alone_returns_diagonal_values,
            test_alignment_is_bottom_right, test_offset_zero_and_column_zero_two_key_mix,
            test_every_offset_is_dense_causal, test_band_of_offsets_is_a_sliding_window,
            test_slash_inside_listed_block_adds_nothing]


def _mutant(key_of):
    def mask(rows, lq, lk, offsets):
        rows = np.asarray(rows, dtype=np.int64)
        out = np.zeros((rows.size, lk), dtype=bool)
        for o in np.asarray(offsets, dtype=np.int64):
            keys = key_of(rows, lq, lk, o)
            ok = (keys >= 0) & (keys < lk)
            out[np.nonzero(ok)[0], keys[ok]] = True
        return out
    return mask


MUTANTS = {
    "above_diagonal": _mutant(lambda r, lq, lk, o: r + (lk - lq) + o),
    "off_by_one": _mutant(lambda r, lq, lk, o: r + (lk - lq) - o - 1),
    "top_left_aligned": _mutant(lambda r, lq, lk, o: r - o),
    "offset_as_key": _mutant(lambda r, lq, lk, o: np.full_like(r, o)),
}


def _intersection_fn(blk_ptr, blk_idx, col_ptr, col_idx, sl_ptr, sl_idx, hq, nqb, lq, lk,
                     block_m=64, block_n=64):
    bc = A.csr_allowed_fn(blk_ptr, blk_idx, col_ptr, col_idx, hq, nqb, lk, block_m, block_n)
    sl_ptr, sl_idx = np.asarray(sl_ptr), np.asarray(sl_idx)

    def fn(b, h, rows):
        c = b * hq + h
        return bc(b, h, rows) & A.slash_row_mask(rows, lq, lk, sl_idx[sl_ptr[c]:sl_ptr[c + 1]])
    return fn


def test_unmutated_oracle_passes_every_pin():
    for pin in _pins():
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS) + ["intersection"])
def test_mutant_is_caught(name, monkeypatch):
    if name == "intersection":
        monkeypatch.setattr(A, "vslash_allowed_fn", _intersection_fn)
    else:
        monkeypatch.setattr(A, "slash_row_mask", MUTANTS[name])
    failed = False
    for pin in _pins():
        try:
            pin()
        except AssertionError:
            failed = True
            break
    assert failed, f"no pin catches the mutant {name}"

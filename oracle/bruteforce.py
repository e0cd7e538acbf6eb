"""Pure-Python brute-force attention for tiny inputs (math.exp, math.fsum, explicit loops).

TEST INFRASTRUCTURE ONLY (see oracle/attention.py). This is the literal definition of
softmax attention written as scalar loops, with no numpy: it pins `oracle.attention` on tiny
shapes. Definition: "Resumen Técnico: FlashMLA-ETAP", section "Mecanismo Central" (S = Q·Kᵀ,
P = softmax(S), O = P·V); GQA sharing from the FAQ of "Activar Flash Attention con llama.cpp
para optimizar la inferencia"; block/column union visibility from the MInference article's
pattern paragraphs. Causal alignment is bottom-right (a reading; the pages are silent).

Inputs are nested Python lists (or anything indexable as x[b][l][h][d]).
"""

from __future__ import annotations

import math


def attention_bruteforce(q, k, v, scale, causal, visible_extra=None):
    """Returns (O[b][i][h][d], LSE[b][h][i]) as nested lists of Python floats.

    visible_extra: None or a function (b, h, i, j) -> bool, ANDed with the causal mask.
    """
    bsz = len(q)
    lq = len(q[0])
    hq = len(q[0][0])
    dqk = len(q[0][0][0])
    lk = len(k[0])
    hkv = len(k[0][0])
    dv = len(v[0][0][0])
    g = hq // hkv
    out = [[[[0.0] * dv for _ in range(hq)] for _ in range(lq)] for _ in range(bsz)]
    lse = [[[0.0] * lq for _ in range(hq)] for _ in range(bsz)]
    for b in range(bsz):
        for h in range(hq):
            kh = h // g
            for i in range(lq):
                scores = []
                for j in range(lk):
                    vis = True
                    if causal and j > i + lk - lq:
                        vis = False
                    if visible_extra is not None and not visible_extra(b, h, i, j):
                        vis = False
                    if vis:
                        dot = math.fsum(float(q[b][i][h][d]) * float(k[b][j][kh][d]) for d in range(dqk))
                        scores.append((j, scale * dot))
                if not scores:
                    lse[b][h][i] = -math.inf
                    continue          # O row stays 0
                mx = max(s for _, s in scores)
                ex = [(j, math.exp(s - mx)) for j, s in scores]
                tot = math.fsum(e for _, e in ex)
                for d in range(dv):
                    out[b][i][h][d] = math.fsum(e * float(v[b][j][kh][d]) for j, e in ex) / tot
                lse[b][h][i] = mx + math.log(tot)
    return out, lse

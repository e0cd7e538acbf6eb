#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

Prints ONE JSON line. The headline is the Llama-3-8B-shaped causal GQA prefill
(B=1, Hq=32, Hkv=8, D=128, L=8192) in attention TFLOP/s, with a roofline object for its
kernel and the fp64 CPU oracle timed on a bounded sample of the same workload. The decode
(GQA 4K, MLA 64K) and block-sparse (128K) workloads are timed in the same run and reported
under "workloads" with their own units (KV-read GB/s, TFLOP/s).

Timing: W untimed warm-up steps, then K steps bracketed by torch.cuda.synchronize(), with
HIP events recorded on the stream the kernels are launched on (torch's current stream).
Inputs are resident in HBM before the timed region starts.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s

HEADLINE = "gqa_prefill_8k"
# The headline's kernel (as rocprofv3 names it) and the sources its machine code comes from.
DENSE_KERNEL = "fwd_dense_kernel<128, 1>"
DENSE_SOURCES = ["fwd_dense.hip", "tile_io.hpp", "common.hpp", "kernels.hpp"]
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------ work counts
def dense_causal_pairs(lq, lk, causal):
    """Visible (query, key) pairs of one head under bottom-right causal masking."""
    if not causal:
        return lq * lk
    off = lk - lq
    tot = 0
    # row i sees min(lk, max(0, i + off + 1)) keys
    import numpy as np
    i = np.arange(lq, dtype=np.int64)
    return int(np.clip(i + off + 1, 0, lk).sum()) if lq else tot


def blocksparse_pairs(lists, B, Hq, L):
    """Exact visible pairs of the block/column union with causal masking (Lq == Lk == L)."""
    import numpy as np
    blk_ptr, blk_idx, col_ptr, col_idx = [np.asarray(x, np.int64) for x in lists]
    nqb = -(-L // 64)
    total = 0
    for bh in range(B * Hq):
        cols = col_idx[col_ptr[bh]:col_ptr[bh + 1]]
        base = bh * nqb
        for qb in range(nqb):
            blks = blk_idx[blk_ptr[base + qb]:blk_ptr[base + qb + 1]]
            r0, r1 = 64 * qb, min(64 * qb + 64, L)            # rows [r0, r1)
            # listed blocks: keys [64kb, 64kb+64) ∩ [0, L), row i sees keys j <= i
            k0 = 64 * blks
            k1 = np.minimum(k0 + 64, L)
            # pairs = sum over rows i of |[k0, k1) ∩ [0, i]|
            rows = np.arange(r0, r1)[:, None]
            total += int(np.clip(np.minimum(k1[None, :], rows + 1) - k0[None, :], 0, None).sum())
            # columns not inside a listed block, each visible to rows i >= c
            inblk = np.isin(cols // 64, blks)
            c = cols[~inblk]
            total += int(np.clip(r1 - np.maximum(c, r0), 0, None).sum())
    return total


def vslash_pairs(slash_ptr, slash_idx, col_ptr, col_idx, B, Hq, L):
    """Exact visible pairs of the column / slash-line union with causal masking (Lq == Lk == L,
    no key blocks): row i sees its columns <= i and keys i - o; a key that is both is counted
    once, and such a pair (c, o) exists for every column c and offset o with c + o < L."""
    import numpy as np
    sp, si, cp, ci = [np.asarray(x, np.int64) for x in (slash_ptr, slash_idx, col_ptr, col_idx)]
    rows = np.arange(L, dtype=np.int64)
    total = 0
    for bh in range(B * Hq):
        offs = np.sort(si[sp[bh]:sp[bh + 1]])
        cols = np.sort(ci[cp[bh]:cp[bh + 1]])
        total += int(np.searchsorted(cols, rows, side="right").sum())
        total += int(np.searchsorted(offs, rows, side="right").sum())
        total -= int(np.searchsorted(offs, L - 1 - cols, side="right").sum())
    return total


# ------------------------------------------------------------------------------ timing
STEP_TIMES = {}   # last time_steps call: per-step event times (ms)


def time_steps(step, steps, warmup):
    """Mean ms per step over `steps` back-to-back steps (HIP events on the launch stream around
    the whole run), and the wall time. A second pass of `steps` steps, each bracketed by its own
    events (recorded without synchronising), gives the spread in STEP_TIMES (p10 / p50 / p90);
    it stays out of the timed run so that those events cannot perturb it."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record(stream)
    for i in range(steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    pick = lambda f: per[min(steps - 1, int(f * (steps - 1) + 0.5))]
    STEP_TIMES.clear()
    STEP_TIMES.update({"ms_p10": round(pick(0.1), 4), "ms_p50": round(pick(0.5), 4),
                       "ms_p90": round(pick(0.9), 4)})
    return start.elapsed_time(end) / steps, wall


def achievable_peaks():
    """Peaks measured on this GPU with library routines, beside the published ones: a bf16 GEMM
    (torch.matmul on contiguous 8192 x 8192 operands, fp32 accumulate) and a 1 GiB device-to-
    device copy (read + write bytes)."""
    import torch
    n = 8192
    g = torch.Generator(device="cuda:0").manual_seed(7)
    a = torch.randn((n, n), device="cuda:0", generator=g).to(torch.bfloat16)
    b = torch.randn((n, n), device="cuda:0", generator=g).to(torch.bfloat16)
    ms, _ = time_steps(lambda: torch.matmul(a, b), 20, 5)
    gemm = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b
    x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(x)
    ms_c, _ = time_steps(lambda: y.copy_(x), 20, 5)
    copy = 2.0 * x.numel() / (ms_c * 1e-3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    return {"bf16_gemm_tflops": round(gemm, 1), "hbm_copy_gbs": round(copy, 1),
            "gemm": "torch.matmul bf16 8192^3", "copy": "1 GiB device copy, read + write"}


def kernel_source_hash(files):
    from sparse_attention_attn_amd.profiling import kernel_source_hash as h
    return h(files)


def load_traffic(workload, src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were taken on
    the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha256_16") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------------------ workloads
def bench_prefill(w, steps, warmup):
    import torch
    import sparse_attention_attn_amd as S
    from workloads import make_qkv
    q, k, v = [t.to("cuda:0") for t in make_qkv(w)]
    o = torch.empty((w.B, w.Lq, w.Hq, w.Dv), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device="cuda:0")
    step = lambda: S.attn_fwd(q, k, v, o, lse, causal=w.causal, scale=w.scale)
    ms, wall = time_steps(step, steps, warmup)
    flops = 2 * (w.Dqk + w.Dv) * w.B * w.Hq * dense_causal_pairs(w.Lq, w.Lk, w.causal)
    return {"ms": ms, "wall_s": wall, "flops": flops, "tflops": flops / (ms * 1e-3) / 1e12,
            **STEP_TIMES}


def bench_decode(w, steps, warmup):
    import torch
    import sparse_attention_attn_amd as S
    from workloads import make_qkv
    q, k, v = make_qkv(w)
    kv_bytes = k.numel() * 2 + (0 if w.mla else v.numel() * 2)
    # rotate >= 1 GiB of KV copies so the 256 MiB Infinity Cache cannot serve repeats
    ncopies = max(2, -(-(1 << 30) // kv_bytes))
    qd = q.to("cuda:0")
    ks = [k.to("cuda:0") for _ in range(ncopies)]
    vs = [t[..., :w.Dv] for t in ks] if w.mla else [v.to("cuda:0") for _ in range(ncopies)]
    o = torch.empty((w.B, w.Lq, w.Hq, w.Dv), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device="cuda:0")
    nsp = S.attn_splitkv_num_splits(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.Dqk, w.Dv)
    # one call per step: split-KV plus the combine (attn_fwd_decode)
    ws = torch.zeros(S.attn_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.Dqk, w.Dv),
                     dtype=torch.uint8, device="cuda:0")
    it = [0]

    def step():
        i = it[0] % ncopies
        it[0] += 1
        S.attn_fwd_decode(qd, ks[i], vs[i], o, lse, causal=w.causal, scale=w.scale, workspace=ws)

    ms, wall = time_steps(step, steps, warmup)
    nbytes = kv_bytes + q.numel() * 2 + o.numel() * 2 + lse.numel() * 4
    return {"ms": ms, "wall_s": wall, "bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9,
            "num_splits": nsp, "kv_copies": ncopies, **STEP_TIMES}


def bench_blocksparse(w, steps, warmup):
    import numpy as np
    import torch
    import sparse_attention_attn_amd as S
    from workloads import make_blocksparse_lists, make_qkv
    q, k, v = [t.to("cuda:0") for t in make_qkv(w)]
    lists = make_blocksparse_lists(w.B, w.Hq, w.Lq, w.Lk, 1000 * w.index + 3)
    dl = [torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0") for x in lists]
    o = torch.empty((w.B, w.Lq, w.Hq, w.Dv), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device="cuda:0")
    step = lambda: S.attn_fwd_blocksparse(q, k, v, o, *dl, lse=lse, causal=True, scale=w.scale)
    ms, wall = time_steps(step, steps, warmup)
    pairs = blocksparse_pairs(lists, w.B, w.Hq, w.Lq)
    flops = 2 * (w.Dqk + w.Dv) * pairs
    dense = w.B * w.Hq * dense_causal_pairs(w.Lq, w.Lk, True)
    res = {"ms": ms, "wall_s": wall, "flops": flops, "tflops": flops / (ms * 1e-3) / 1e12,
           "density_vs_causal": pairs / dense, **STEP_TIMES}
    # The same attention with lists built from Q and K at run time (attn_build_sparse_index:
    # 96 blocks per query block, 1000 columns per head, about the synthetic lists' density).
    topk, ncols = 96, 1000
    nb, nc = S.attn_sparse_index_sizes(w.B, w.Hq, w.Lq, topk, ncols)
    nqb = -(-w.Lq // 64)
    outs = (torch.empty(w.B * w.Hq * nqb + 1, dtype=torch.int32, device="cuda:0"),
            torch.empty(nb, dtype=torch.int32, device="cuda:0"),
            torch.empty(w.B * w.Hq + 1, dtype=torch.int32, device="cuda:0"),
            torch.empty(nc, dtype=torch.int32, device="cuda:0"))
    ws = torch.empty(S.attn_sparse_index_workspace_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Dqk),
                     dtype=torch.uint8, device="cuda:0")
    build = lambda: S.attn_build_sparse_index(q, k, topk, ncols, scale=w.scale, outputs=outs,
                                              workspace=ws)
    ms_b, _ = time_steps(build, steps, warmup)
    built = build()
    torch.cuda.synchronize()
    step_d = lambda: (build(), S.attn_fwd_blocksparse(q, k, v, o, *built, lse=lse, causal=True,
                                                      scale=w.scale))
    ms_d, _ = time_steps(step_d, steps, warmup)
    hl = [t.cpu().numpy() for t in built]
    pairs_d = blocksparse_pairs(hl, w.B, w.Hq, w.Lq)
    flops_d = 2 * (w.Dqk + w.Dv) * pairs_d
    res["dynamic"] = {"index_build_ms": round(ms_b, 4), "build_plus_attention_ms": round(ms_d, 4),
                      "topk_blocks": topk, "n_cols": ncols,
                      "density_vs_causal": round(pairs_d / dense, 4),
                      "tflops_incl_build": round(flops_d / (ms_d * 1e-3) / 1e12, 3)}
    return res


def bench_vslash(w, steps, warmup):
    import numpy as np
    import torch
    import sparse_attention_attn_amd as S
    from workloads import make_qkv, make_vslash_lists
    q, k, v = [t.to("cuda:0") for t in make_qkv(w)]
    sp, si, cp, ci = make_vslash_lists(w.B, w.Hq, w.Lk, 1000 * w.index + 3)
    nqb = -(-w.Lq // 64)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda:0")
    bp, bi = dev(np.zeros(w.B * w.Hq * nqb + 1)), dev(np.zeros(0))
    dsp, dsi, dcp, dci = dev(sp), dev(si), dev(cp), dev(ci)
    o = torch.empty((w.B, w.Lq, w.Hq, w.Dv), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(S.attn_vertical_slash_workspace_bytes(w.B, w.Hq, w.Lk), dtype=torch.uint8,
                     device="cuda:0")
    step = lambda: S.attn_fwd_vertical_slash(q, k, v, o, bp, bi, dcp, dci, dsp, dsi, lse=lse,
                                             causal=True, scale=w.scale, workspace=ws)
    ms, wall = time_steps(step, steps, warmup)
    pairs = vslash_pairs(sp, si, cp, ci, w.B, w.Hq, w.Lq)
    flops = 2 * (w.Dqk + w.Dv) * pairs
    dense = w.B * w.Hq * dense_causal_pairs(w.Lq, w.Lk, True)
    res = {"ms": ms, "wall_s": wall, "flops": flops, "tflops": flops / (ms * 1e-3) / 1e12,
           "density_vs_causal": pairs / dense, **STEP_TIMES}
    # Lists built from Q and K at run time (attn_build_vslash_index), as many columns and lines
    # as the synthetic lists. Random inputs have no diagonal structure, so the chosen lines
    # scatter over all offsets and the forward then visits nearly every causal block.
    ncols, nslash = 1000, int(sp[1] - sp[0])
    nc, ns = w.B * w.Hq * min(ncols, w.Lk), w.B * w.Hq * min(nslash, w.Lk)
    outs = (torch.empty(w.B * w.Hq + 1, dtype=torch.int32, device="cuda:0"),
            torch.empty(nc, dtype=torch.int32, device="cuda:0"),
            torch.empty(w.B * w.Hq + 1, dtype=torch.int32, device="cuda:0"),
            torch.empty(ns, dtype=torch.int32, device="cuda:0"))
    iws = torch.empty(S.attn_sparse_index_workspace_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Dqk),
                      dtype=torch.uint8, device="cuda:0")
    build = lambda: S.attn_build_vslash_index(q, k, ncols, nslash, scale=w.scale, outputs=outs,
                                              workspace=iws)
    ms_b, _ = time_steps(build, steps, warmup)
    bcp, bci, bsp, bsi = build()
    step_d = lambda: (build(), S.attn_fwd_vertical_slash(q, k, v, o, bp, bi, bcp, bci, bsp, bsi,
                                                         lse=lse, causal=True, scale=w.scale,
                                                         workspace=ws))
    ms_d, _ = time_steps(step_d, 2, 1)
    hl = [t.cpu().numpy() for t in (bsp, bsi, bcp, bci)]
    pairs_d = vslash_pairs(*hl, w.B, w.Hq, w.Lq)
    res["dynamic"] = {"index_build_ms": round(ms_b, 4), "build_plus_attention_ms": round(ms_d, 4),
                      "n_cols": ncols, "n_slash": nslash,
                      "density_vs_causal": round(pairs_d / dense, 4),
                      "tflops_incl_build": round(2 * (w.Dqk + w.Dv) * pairs_d / (ms_d * 1e-3)
                                                 / 1e12, 3)}
    return res


def mla_causal_pairs(lq, lk):
    """Visible (query, key) pairs of one head with bottom-right causal masking."""
    return sum(max(0, min(lk, p + lk - lq + 1)) for p in range(lq))


def bench_etap_grid(steps, warmup):
    """The FlashMLA-ETAP decode grid: MLA (16 heads, Dqk 576, V = first 512 columns of the
    latent cache), batch 16 and 32, one or two query tokens, KV length 512..64K, split-KV +
    LSE combine per step. Inputs are drawn on the device from seeded generators (the largest
    points hold several GB); KV copies rotate over >= 1 GiB so the 256 MB Infinity Cache
    cannot serve repeats."""
    import torch
    import sparse_attention_attn_amd as S
    from workloads import ETAP_GRID, randn_bf16_device
    out = []
    caches = {}
    for name, w in ETAP_GRID.items():
        key = (w.B, w.Lk)
        kv_bytes = w.B * w.Lk * w.Dqk * 2
        if key not in caches:
            caches.clear()
            torch.cuda.empty_cache()
            ncopies = max(2, -(-(1 << 30) // kv_bytes))
            caches[key] = [randn_bf16_device((w.B, w.Lk, 1, w.Dqk), 1000 * w.index + 1 + 7 * c)
                           for c in range(ncopies)]
        ks = caches[key]
        q = randn_bf16_device((w.B, w.Lq, w.Hq, w.Dqk), 1000 * w.index)
        o = torch.empty((w.B, w.Lq, w.Hq, w.Dv), dtype=torch.bfloat16, device="cuda:0")
        lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device="cuda:0")
        nsp = S.attn_splitkv_num_splits(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.Dqk, w.Dv)
        op = torch.empty((nsp, w.B, w.Hq, w.Lq, w.Dv), dtype=torch.float32, device="cuda:0")
        lp = torch.empty((nsp, w.B, w.Hq, w.Lq), dtype=torch.float32, device="cuda:0")
        it = [0]

        def step():
            kk = ks[it[0] % len(ks)]
            it[0] += 1
            S.attn_fwd_splitkv(q, kk, kk[..., :w.Dv], op, lp, causal=True, scale=w.scale)
            S.attn_combine_lse(op, lp, o, lse)

        ms, _ = time_steps(step, steps, warmup)
        flops = 2 * (w.Dqk + w.Dv) * w.B * w.Hq * mla_causal_pairs(w.Lq, w.Lk)
        nbytes = kv_bytes + q.numel() * 2 + o.numel() * 2 + lse.numel() * 4
        out.append({"B": w.B, "Lq": w.Lq, "Lk": w.Lk, "num_splits": nsp, "us": round(ms * 1e3, 2),
                    "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                    "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)})
        log(f"  {name}: {out[-1]}")
    caches.clear()
    return out


def bench_memory(lengths, eager_max):
    """Peak device memory of one causal prefill (B 1, Hq 32, Hkv 8, D 128) above its inputs and
    outputs: attn_fwd's (it allocates nothing and keeps no S or P) against an eager attention
    that materialises the scores (fp32 S = Q·Kᵀ, softmax, P·V in plain PyTorch). The eager one
    is measured up to `eager_max` keys; its 2·Hq·L²·4 bytes of S and P are given beyond."""
    import torch
    import sparse_attention_attn_amd as S
    from workloads import randn_bf16_device
    B, Hq, Hkv, D = 1, 32, 8, 128
    scale = D ** -0.5
    out = []
    for L in lengths:
        torch.cuda.empty_cache()
        q = randn_bf16_device((B, L, Hq, D), 900 + L)
        k = randn_bf16_device((B, L, Hkv, D), 901 + L)
        v = randn_bf16_device((B, L, Hkv, D), 902 + L)
        o = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device="cuda:0")
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda:0")
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        S.attn_fwd(q, k, v, o, lse, causal=True, scale=scale)
        torch.cuda.synchronize()
        ours = torch.cuda.max_memory_allocated() - base
        io = sum(t.numel() * t.element_size() for t in (q, k, v, o, lse))
        rec = {"L": L, "inputs_outputs_bytes": int(io), "allocated_before_bytes": int(base),
               "attn_fwd_extra_bytes": int(ours),
               "eager_extra_bytes_formula": 2 * B * Hq * L * L * 4}
        if L <= eager_max:
            g = Hq // Hkv
            qf = q.float().permute(0, 2, 1, 3).contiguous()
            kf = k.float().repeat_interleave(g, dim=2).permute(0, 2, 3, 1).contiguous()
            vf = v.float().repeat_interleave(g, dim=2).permute(0, 2, 1, 3).contiguous()
            torch.cuda.synchronize()
            base_e = torch.cuda.memory_allocated()
            torch.cuda.reset_peak_memory_stats()
            s_ = torch.matmul(qf, kf)
            s_.mul_(scale)
            s_.masked_fill_(torch.ones(L, L, dtype=torch.bool, device="cuda:0").triu_(1),
                            float("-inf"))
            p_ = torch.softmax(s_, dim=-1)
            del s_
            oe = torch.matmul(p_, vf)
            torch.cuda.synchronize()
            rec["eager_extra_bytes_measured"] = int(torch.cuda.max_memory_allocated() - base_e)
            del p_, oe, qf, kf, vf
        out.append(rec)
        log(f"  memory L={L}: {rec}")
        del q, k, v, o, lse
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------------------ CPU baseline
def cpu_baseline(w, budget_s):
    """The fp64 oracle, as it stands, timed on a bounded sample of the headline workload:
    whole query heads (every row, all visible keys), one after another until about `budget_s`
    of CPU work or the whole workload is done."""
    import numpy as np
    from oracle import attention as A
    from workloads import make_qkv, sampled_rows
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    q, k, v = make_qkv(w)
    qf = q.float().numpy().astype(np.float64)
    kf = k.float().numpy().astype(np.float64)
    vf = v.float().numpy().astype(np.float64)
    sc = A.effective_scale(w.scale)
    rows = sampled_rows(w.Lq, w.Lq, 1000 * w.index + 4, edge=64)
    per_row_pairs = np.clip(rows + (w.Lk - w.Lq) + 1, 0, w.Lk).sum()
    t0 = time.perf_counter()
    heads = 0
    while True:
        A.attention_rows(qf, kf, vf, sc, w.causal, 0, heads % w.Hq, rows)
        heads += 1
        if time.perf_counter() - t0 >= budget_s or heads >= w.Hq:
            break
    el = time.perf_counter() - t0
    flops = 2 * (w.Dqk + w.Dv) * int(per_row_pairs) * heads
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{heads} of {w.Hq} query head(s) x {len(rows)} of {w.Lq} rows of "
                      f"{w.name}, all visible keys, fp64 numpy; {el:.1f} s"}


# ------------------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default=None, help="comma list of workloads to run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-etap-grid", action="store_true",
                    help="skip the FlashMLA-ETAP decode grid sweep")
    ap.add_argument("--no-memory", action="store_true",
                    help="skip the peak-memory comparison at long sequence lengths")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the bf16 GEMM / device copy measurement of achievable peaks")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(this attention path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from workloads import WORKLOADS

    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes read + {n} bytes written")
        del src, dst

    names = args.only.split(",") if args.only else list(WORKLOADS)
    res = {}
    for name in names:
        w = WORKLOADS[name]
        log(f"workload {name}: {w}")
        if w.kind == "prefill":
            res[name] = bench_prefill(w, args.steps if name == HEADLINE else max(3, args.steps // 4),
                                      args.warmup)
        elif w.kind in ("decode", "mla_decode"):
            res[name] = bench_decode(w, args.steps * 5, args.warmup)
        elif w.kind == "blocksparse":
            res[name] = bench_blocksparse(w, max(3, args.steps // 4), min(args.warmup, 2))
        elif w.kind == "vslash":
            res[name] = bench_vslash(w, max(3, args.steps // 4), min(args.warmup, 2))
        log(f"  -> {res[name]}")

    head = WORKLOADS[HEADLINE]
    out = {
        "metric": "attention TFLOP/s (prefill) and KV-read GB/s (decode), % of MI355X peak",
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
    }
    if HEADLINE in res:
        r = res[HEADLINE]
        src_hash = kernel_source_hash(DENSE_SOURCES)
        out.update({
            "value": round(r["tflops"], 3),
            "ms_per_step": round(r["ms"], 4),
            "config": {"workload": HEADLINE, "B": head.B, "Hq": head.Hq, "Hkv": head.Hkv,
                       "seq_len": head.Lq, "head_dim": head.Dqk, "causal": head.causal,
                       "flops_per_step": r["flops"]},
            "roofline": {"bound": "mfma", "achieved": round(r["tflops"], 3),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(r["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": load_traffic(HEADLINE, src_hash),
                         "kernel": DENSE_KERNEL,
                         "kernel_source_sha256_16": src_hash},
        })
    ach = None
    if not args.no_achievable:
        log("achievable peaks (bf16 GEMM, device copy) ...")
        ach = achievable_peaks()
        out["achievable_peaks"] = ach
        if HEADLINE in res:
            out["roofline"]["frac_of_achievable"] = round(res[HEADLINE]["tflops"] /
                                                          ach["bf16_gemm_tflops"], 4)
    wl = {}
    for name, r in res.items():
        pct = {kk: r[kk] for kk in ("ms_p10", "ms_p50", "ms_p90") if kk in r}
        if "gbs" in r:
            wl[name] = {"value": round(r["gbs"], 1), "unit": "GB/s", "ms": round(r["ms"], 4),
                        **pct, "frac_of_hbm_peak": round(r["gbs"] / HBM_PEAK_GBS, 4),
                        "num_splits": r["num_splits"], "bytes": r["bytes"]}
            if ach:
                wl[name]["frac_of_achievable"] = round(r["gbs"] / ach["hbm_copy_gbs"], 4)
        else:
            wl[name] = {"value": round(r["tflops"], 3), "unit": "TFLOP/s", "ms": round(r["ms"], 4),
                        **pct, "frac_of_mfma_peak": round(r["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
                        "flops": r["flops"]}
            if ach:
                wl[name]["frac_of_achievable"] = round(r["tflops"] / ach["bf16_gemm_tflops"], 4)
            if "density_vs_causal" in r:
                wl[name]["density_vs_causal"] = round(r["density_vs_causal"], 4)
            if "dynamic" in r:
                wl[name]["dynamic_index"] = r["dynamic"]
    out["workloads"] = wl
    if not args.no_etap_grid and args.only is None:
        log("FlashMLA-ETAP decode grid ...")
        out["etap_grid"] = {"unit": "split-KV + combine per step; TFLOP/s = 2*(576+512) per "
                                    "visible (query, key) pair; GB/s = latent cache + Q + O + LSE",
                            "points": bench_etap_grid(max(5, args.steps // 2), 3)}
    if not args.no_memory and args.only is None:
        log("peak memory at long sequence lengths ...")
        out["memory"] = {"op": "causal prefill B 1, Hq 32, Hkv 8, D 128",
                         "points": bench_memory([4096, 8192, 16384, 32768, 65536, 131072],
                                                eager_max=16384)}
    if not args.no_cpu_baseline and HEADLINE in res:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(head, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

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
DENSE_KERNEL = "fwd_dense_kernel<128, 1, 8, false>"
DENSE_SOURCES = ["fwd_dense.hip", "tile_io.hpp", "common.hpp", "kernels.hpp"]
# The sparse prefill kernels (block-sparse and vertical-slash) and their sources: their figure of
# merit beside the MFMA fraction is the rate of their L2-miss traffic against the read ceiling.
SPARSE_SOURCES = ["fwd_blocksparse.hip", "tile_io.hpp", "common.hpp", "kernels.hpp"]
SPARSE_WORKLOADS = ("blocksparse_128k", "vslash_128k")
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


MIN_WARMUP_S = 0.3   # set from --min-warmup-ms


def time_steps(step, steps, warmup):
    """Mean ms per step over `steps` back-to-back steps (HIP events on the launch stream around
    the whole run), and the wall time. A second pass of `steps` steps, each bracketed by its own
    events (recorded without synchronising), gives the spread in STEP_TIMES (p10 / p50 / p90);
    it stays out of the timed run so that those events cannot perturb it.

    Warm-up: `warmup` untimed steps, continued (untimed, same step) until at least MIN_WARMUP_S
    of wall time has passed. The GPU raises its clock over the first few milliseconds of work:
    timed right after 5 steps of the 8K prefill (3 ms), the 20-step mean ran about 10% slower
    than the same steps after 300 ms, whose mean matches the per-step p50 of the second pass.
    STEP_TIMES records how many warm-up steps ran."""
    import torch
    t0 = time.perf_counter()
    n_warm = 0
    while n_warm < warmup or time.perf_counter() - t0 < MIN_WARMUP_S:
        step()
        n_warm += 1
        if n_warm >= warmup and n_warm % 8 == 0:
            torch.cuda.synchronize()
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
                       "ms_p90": round(pick(0.9), 4), "warmup_steps_run": n_warm})
    return start.elapsed_time(end) / steps, wall


def achievable_peaks():
    """Peaks measured on this GPU, beside the published ones: a bf16 GEMM (torch.matmul on
    contiguous 8192 x 8192 operands, fp32 accumulate), a 1 GiB device-to-device copy (read +
    write bytes), and the probe library's read ceilings and MFMA stream. frac_of_achievable
    divides by the higher of the GEMM and the MFMA stream, and by the best HBM read ceiling."""
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
    out = {"bf16_gemm_tflops": round(gemm, 1), "hbm_copy_gbs": round(copy, 1),
           "gemm": "torch.matmul bf16 8192^3", "copy": "1 GiB device copy, read + write"}
    try:
        out["read_ceilings"] = read_ceilings()
        out["mfma_stream"] = mfma_stream()
    except OSError as e:  # the probe library was not built: report it, keep the rest
        out["read_ceilings"] = {"error": f"libattn_probes.so not loaded ({e})"}
    # the ceilings the kernels are held against: the matrix cores' sustained rate on random
    # operands (above what the library GEMM reaches), and the best HBM read rate (decode only
    # reads; a copy also writes)
    ms_ = out.get("mfma_stream", {}).get("tflops")
    out["achievable_mfma_tflops"] = max(gemm, ms_) if ms_ else round(gemm, 1)
    rc = out["read_ceilings"]
    reads = [rc[k] for k in ("hbm_stream_read_gbs", "hbm_tile_gather_read_gbs",
                             "hbm_stream_nt_read_gbs", "hbm_tile_gather_nt_read_gbs") if k in rc]
    out["achievable_hbm_read_gbs"] = max(reads) if reads else round(copy, 1)
    return out


def mfma_stream():
    """The bf16 MFMA rate this GPU sustains on random operands (libattn_probes.so
    probe_mfma_stream: 1024 workgroups of 8 waves, each wave 32 MFMAs 32x32x16 per round on 8
    operand pairs and 4 accumulator chains)."""
    import torch
    lib = _probe_lib()
    grid, iters = 1024, 1000
    g = torch.Generator(device="cuda:0").manual_seed(13)
    ops = torch.randn(16 * 64 * 8, device="cuda:0", generator=g).to(torch.bfloat16)
    sink = torch.zeros(grid * 512, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream

    def step():
        rc = lib.probe_mfma_stream(ops.data_ptr(), grid, iters, sink.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"MFMA probe launch failed: hipError {rc}")

    ms, _ = time_steps(step, 10, 3)
    flops = grid * 8 * iters * 32 * 32768
    return {"tflops": round(flops / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 4),
            "probe": "probe_mfma_stream: 1024 x 8 waves x 1000 rounds x 32 MFMA 32x32x16 bf16, "
                     "random operands"}


def _probe_lib():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_attn_amd", "libattn_probes.so"))
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.probe_read_tiles.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    lib.probe_read_tiles.restype = i32
    lib.probe_read_rows.argtypes = [vp, vp, vp, i32, i32, i32, ctypes.c_int64, vp, vp]
    lib.probe_read_rows.restype = i32
    lib.probe_read_tiles_nt.argtypes = lib.probe_read_tiles.argtypes
    lib.probe_read_tiles_nt.restype = i32
    lib.probe_read_rows_nt.argtypes = lib.probe_read_rows.argtypes
    lib.probe_read_rows_nt.restype = i32
    lib.probe_mfma_stream.argtypes = [vp, i32, i32, vp, vp]
    lib.probe_mfma_stream.restype = i32
    return lib


def read_ceilings():
    """Read rates of this GPU measured with the library's own probe kernel (libattn_probes.so):
    whole 32 KiB tiles (the K and V bytes of one 64-key tile at D = 128), read in order
    (a stream: each XCD reads distinct tiles) or at seeded random tile positions, from a 2 GiB
    region (HBM) and from a 128 MiB region re-read launch after launch (two KV heads' K and V
    at 128K keys: larger than the eight 4 MiB L2s, inside the 256 MiB Infinity Cache).
    2048 workgroups of 256 lanes, each reading 16 tiles one after another. The HBM reads are
    also measured with the non-temporal cache policy (the decode kernels' copies use it)."""
    import torch
    lib = _probe_lib()
    grid, per_wg, tile = 2048, 16, 32 << 10
    ntile = grid * per_wg
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(grid * 256, dtype=torch.int32, device="cuda:0")
    g = torch.Generator().manual_seed(11)
    res = {}
    for region_name, region, steps in (("hbm", 2 << 30, 20), ("infinity_cache", 128 << 20, 50)):
        buf = torch.empty(region, dtype=torch.uint8, device="cuda:0")
        nreg = region // tile
        kinds = ("stream", "tile_gather", "stream_nt", "tile_gather_nt") if region_name == "hbm" \
            else ("stream", "tile_gather")
        for kind in kinds:
            probe = lib.probe_read_tiles_nt if kind.endswith("_nt") else lib.probe_read_tiles
            if kind.startswith("stream"):
                # workgroup g (XCD g % 8) reads 16 consecutive tiles; the XCDs start 1/8 of the
                # region apart, so no XCD reads a tile twice in a launch (its L2 never hits)
                g_ = torch.arange(grid, dtype=torch.int64).repeat_interleave(per_wg)
                t_ = torch.arange(per_wg, dtype=torch.int64).repeat(grid)
                ids = (((g_ // 8) * per_wg + t_ + (g_ % 8) * (nreg // 8)) % nreg).to(torch.int32)
            else:
                ids = torch.randint(0, nreg, (ntile,), generator=g, dtype=torch.int32)
            ids = ids.to("cuda:0")

            def step():
                rc = probe(buf.data_ptr(), ids.data_ptr(), per_wg, grid, tile,
                           sink.data_ptr(), stream)
                if rc != 0:
                    raise RuntimeError(f"read probe launch failed: hipError {rc}")

            ms, _ = time_steps(step, steps, 10)
            res[f"{region_name}_{kind}_read_gbs"] = round(ntile * tile / (ms * 1e-3) / 1e9, 1)
            del ids
        del buf
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    res["probe"] = ("libattn_probes.so: 2048 x 256 lanes, 16 tiles of 32 KiB each, 16-byte "
                    "loads, 8 in flight per lane")
    return res


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
    times = dict(STEP_TIMES)
    nbytes = kv_bytes + q.numel() * 2 + o.numel() * 2 + lse.numel() * 4
    try:
        floor = decode_read_floor(w, nsp, ks, None if w.mla else vs, kv_bytes, steps, warmup)
    except OSError as e:  # the probe library was not built: report it, keep the rest
        floor = {"error": f"libattn_probes.so not loaded ({e})"}
    return {"ms": ms, "wall_s": wall, "bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9,
            "num_splits": nsp, "kv_copies": ncopies, "read_floor": floor, **times}


def decode_read_floor(w, nsp, ks, vs, kv_bytes, steps, warmup):
    """The time a plain read of exactly the cache rows the split kernel reads takes
    (libattn_probes.so `probe_read_rows`): one workgroup per (batch, split, KV head) in the split
    kernel's order (KV head fastest), each reading its split's K rows (and V rows, unless V is
    the latent itself) with 16-byte loads, over the same KV copies in the same rotation. It has
    no softmax, no MFMA, no LDS and no combine, so the decode step's time over it is what the
    kernels add to moving the bytes. Only for shapes whose workgroups each take one column block
    and a whole split of visible keys (None otherwise)."""
    import torch
    g = w.Hq // w.Hkv
    chunk = 64 * -(-(-(-w.Lk // nsp)) // 64)
    if g * w.Lq > 16 or w.Lk % chunk or (w.causal and w.Lq > 1) or (vs and w.Dv != w.Dqk):
        return None
    lib = _probe_lib()
    lid = torch.arange(w.B * nsp * w.Hkv, dtype=torch.int64)
    hkv, sp, b = lid % w.Hkv, (lid // w.Hkv) % nsp, lid // (w.Hkv * nsp)
    row_bytes, stride = w.Dqk * 2, w.Hkv * w.Dqk * 2
    base = (((b * w.Lk + sp * chunk) * w.Hkv + hkv) * row_bytes).to("cuda:0")
    sink = torch.zeros(lid.numel() * 256, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    for t in ks + (vs or []):
        assert t.is_contiguous() and t.shape == (w.B, w.Lk, w.Hkv, w.Dqk)
    it = [0]

    def timed(probe):
        def step():
            i = it[0] % len(ks)
            it[0] += 1
            rc = probe(ks[i].data_ptr(), vs[i].data_ptr() if vs else None, base.data_ptr(),
                       lid.numel(), chunk, row_bytes, stride, sink.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError(f"read probe launch failed: hipError {rc}")
        ms, _ = time_steps(step, steps, warmup)
        return ms

    # the split kernel's copies take the non-temporal policy; the default policy for reference
    ms = timed(lib.probe_read_rows_nt)
    ms_default = timed(lib.probe_read_rows)
    return {"ms": round(ms, 4), "kv_gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 1),
            "ms_default_policy": round(ms_default, 4),
            "probe": (f"probe_read_rows_nt: {lid.numel()} workgroups x {chunk} rows of "
                      f"{row_bytes} B at stride {stride} B" +
                      (", K and V" if vs else ", latent only") + ", non-temporal loads")}


def bench_blocksparse(w, steps, warmup, dynamic=True):
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
    if not dynamic:
        return res
    # The same attention with lists built from Q and K at run time (attn_build_sparse_index:
    # 96 blocks per query block, 1000 columns per head, about the synthetic lists' density),
    # on the workload's noise inputs (nothing for the builder to find) and on inputs with a
    # planted band and planted columns (make_structured_qk).
    from workloads import make_structured_qk
    topk, ncols = 96, 1000
    nb, nc = S.attn_sparse_index_sizes(w.B, w.Hq, w.Lq, topk, ncols)
    nqb = -(-w.Lq // 64)
    outs = (torch.empty(w.B * w.Hq * nqb + 1, dtype=torch.int32, device="cuda:0"),
            torch.empty(nb, dtype=torch.int32, device="cuda:0"),
            torch.empty(w.B * w.Hq + 1, dtype=torch.int32, device="cuda:0"),
            torch.empty(nc, dtype=torch.int32, device="cuda:0"))
    ws = torch.empty(S.attn_sparse_index_workspace_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Dqk),
                     dtype=torch.uint8, device="cuda:0")

    def dynamic(qd, kd, inputs):
        build = lambda: S.attn_build_sparse_index(qd, kd, topk, ncols, scale=w.scale,
                                                  outputs=outs, workspace=ws)
        ms_b, _ = time_steps(build, steps, warmup)
        built = build()
        torch.cuda.synchronize()
        step_d = lambda: (build(), S.attn_fwd_blocksparse(qd, kd, v, o, *built, lse=lse,
                                                          causal=True, scale=w.scale))
        ms_d, _ = time_steps(step_d, steps, warmup)
        hl = [t.cpu().numpy() for t in built]
        pairs_d = blocksparse_pairs(hl, w.B, w.Hq, w.Lq)
        flops_d = 2 * (w.Dqk + w.Dv) * pairs_d
        return {"inputs": inputs, "index_build_ms": round(ms_b, 4),
                "build_plus_attention_ms": round(ms_d, 4), "topk_blocks": topk, "n_cols": ncols,
                "density_vs_causal": round(pairs_d / dense, 4),
                "tflops_incl_build": round(flops_d / (ms_d * 1e-3) / 1e12, 3)}

    res["dynamic"] = dynamic(q, k, "the workload's Q and K (N(0, 1) noise: no structure)")
    qs, kst = make_structured_qk(w.B, w.Lq, w.Hq, w.Hkv, w.Dqk, 1000 * w.index + 5, window=6144,
                                 scale=w.scale)
    res["dynamic_structured"] = dynamic(
        qs, kst, "make_structured_qk: noise plus a planted band (window 6144, rise 6) and 1000 "
                 "planted columns per KV head (rise 8)")
    del qs, kst
    return res


def bench_vslash(w, steps, warmup, dynamic=True):
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
    if not dynamic:
        return res
    # Lists built from Q and K at run time (attn_build_vslash_index), as many columns and lines
    # as the synthetic lists. On the workload's noise inputs the chosen lines scatter over all
    # offsets (the forward then reads a K/V window per line and row block); on inputs with a
    # planted band and planted columns (make_structured_qk) they gather in the band.
    from workloads import make_structured_qk
    ncols, nslash = 1000, int(sp[1] - sp[0])
    nc, ns = w.B * w.Hq * min(ncols, w.Lk), w.B * w.Hq * min(nslash, w.Lk)
    outs = (torch.empty(w.B * w.Hq + 1, dtype=torch.int32, device="cuda:0"),
            torch.empty(nc, dtype=torch.int32, device="cuda:0"),
            torch.empty(w.B * w.Hq + 1, dtype=torch.int32, device="cuda:0"),
            torch.empty(ns, dtype=torch.int32, device="cuda:0"))
    iws = torch.empty(S.attn_sparse_index_workspace_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Dqk),
                      dtype=torch.uint8, device="cuda:0")

    def dynamic(qd, kd, inputs, steps_d):
        build = lambda: S.attn_build_vslash_index(qd, kd, ncols, nslash, scale=w.scale,
                                                  outputs=outs, workspace=iws)
        ms_b, _ = time_steps(build, steps, warmup)
        bcp, bci, bsp, bsi = build()
        step_d = lambda: (build(), S.attn_fwd_vertical_slash(qd, kd, v, o, bp, bi, bcp, bci, bsp,
                                                             bsi, lse=lse, causal=True,
                                                             scale=w.scale, workspace=ws))
        ms_d, _ = time_steps(step_d, steps_d, 1)
        hl = [t.cpu().numpy() for t in (bsp, bsi, bcp, bci)]
        pairs_d = vslash_pairs(*hl, w.B, w.Hq, w.Lq)
        return {"inputs": inputs, "index_build_ms": round(ms_b, 4),
                "build_plus_attention_ms": round(ms_d, 4), "n_cols": ncols, "n_slash": nslash,
                "density_vs_causal": round(pairs_d / dense, 4),
                "tflops_incl_build": round(2 * (w.Dqk + w.Dv) * pairs_d / (ms_d * 1e-3) / 1e12,
                                           3)}

    res["dynamic"] = dynamic(q, k, "the workload's Q and K (N(0, 1) noise: no structure)", 2)
    # A band rise of 12 that stays above 10 over the first ~1100 offsets (window 4096), over
    # scores whose noise has a standard deviation near 1.8: the probe's diagonal sums then rank
    # those offsets above nearly every offset that only a noise extreme or a planted column
    # crosses, as in the static lists' 1024-offset band (at 32K keys, checked with the oracle's
    # builder: 1079 of the 1088 lines below offset 1500). With a band that halves by offset
    # 1024 (window 2048), a few hundred such offsets enter the lines and run as windows.
    qs, kst = make_structured_qk(w.B, w.Lq, w.Hq, w.Hkv, w.Dqk, 1000 * w.index + 5, window=4096,
                                 band_logit=12.0, col_logit=5.0, scale=w.scale)
    res["dynamic_structured"] = dynamic(
        qs, kst, "make_structured_qk: noise plus a planted band (window 4096, rise 12) and 1000 "
                 "planted columns per KV head (rise 5)", steps)
    del qs, kst
    return res


def mla_causal_pairs(lq, lk):
    """Visible (query, key) pairs of one head with bottom-right causal masking."""
    return sum(max(0, min(lk, p + lk - lq + 1)) for p in range(lq))


def bench_etap_grid(steps, warmup):
    """The FlashMLA-ETAP decode grid: MLA (16 heads, Dqk 576, V = first 512 columns of the
    latent cache), batch 16 and 32, one or two query tokens, KV length 512..64K, split-KV +
    LSE combine per step (one attn_fwd_decode call). Inputs are drawn on the device from
    seeded generators (the largest points hold several GB); KV copies rotate over >= 1 GiB so
    the 256 MB Infinity Cache cannot serve repeats."""
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
        ws = torch.empty(max(256, S.attn_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Lk,
                                                                  w.Dqk, w.Dv)),
                         dtype=torch.uint8, device="cuda:0")
        kv = [(kk, kk[..., :w.Dv]) for kk in ks]  # V views made once, not per step
        it = [0]

        # one library call per step: split-KV and the combine (attn_fwd_decode), so the short
        # caches are not timed on the binding's per-call host work twice
        def step():
            kk, vv = kv[it[0] % len(kv)]
            it[0] += 1
            S.attn_fwd_decode(q, kk, vv, o, lse, causal=True, scale=w.scale, workspace=ws)

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


def bench_prefill_sweep(shapes, steps=10, warmup=3):
    """Causal GQA prefill (attn_fwd, D 128) over batch, head counts and lengths other than the
    headline's, including grids of one round or less (where the launcher takes the 128-row
    workgroup form). Inputs: seeded device N(0, 1) in bf16."""
    import torch
    import sparse_attention_attn_amd as S
    from workloads import randn_bf16_device
    out = []
    for (B, Hq, Hkv, L) in shapes:
        D = 128
        q = randn_bf16_device((B, L, Hq, D), 7100 + L)
        k = randn_bf16_device((B, L, Hkv, D), 7101 + L)
        v = randn_bf16_device((B, L, Hkv, D), 7102 + L)
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda:0")
        ms, _ = time_steps(lambda: S.attn_fwd(q, k, v, o, lse, causal=True, scale=D ** -0.5),
                           steps, warmup)
        flops = 2 * 2 * D * B * Hq * dense_causal_pairs(L, L, True)
        out.append({"B": B, "Hq": Hq, "Hkv": Hkv, "L": L, "ms": round(ms, 4),
                    "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                    "workgroups_256_rows": B * Hq * (-(-L // 256))})
        del q, k, v, o, lse
    torch.cuda.empty_cache()
    return out


def bench_chunked_prefill(shapes, steps=10, warmup=3):
    """A query chunk against a longer cache (bottom-right causal, D 128): attn_fwd (one
    workgroup per 128 or 256 rows of a head) against the one-call split-KV path
    (attn_fwd_decode, which runs the prefill kernel over split key ranges and the LSE combine).
    Inputs: seeded device N(0, 1) in bf16."""
    import torch
    import sparse_attention_attn_amd as S
    from workloads import randn_bf16_device
    out = []
    for (B, Hq, Hkv, Lq, Lk) in shapes:
        D = 128
        q = randn_bf16_device((B, Lq, Hq, D), 7200 + Lq)
        k = randn_bf16_device((B, Lk, Hkv, D), 7201 + Lk)
        v = randn_bf16_device((B, Lk, Hkv, D), 7202 + Lk)
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device="cuda:0")
        ws = torch.empty(max(256, S.attn_decode_workspace_bytes(B, Hq, Hkv, Lq, Lk, D, D)),
                         dtype=torch.uint8, device="cuda:0")
        ms_f, _ = time_steps(lambda: S.attn_fwd(q, k, v, o, lse, causal=True), steps, warmup)
        ms_s, _ = time_steps(lambda: S.attn_fwd_decode(q, k, v, o, lse, causal=True,
                                                       workspace=ws), steps, warmup)
        flops = 2 * 2 * D * B * Hq * dense_causal_pairs(Lq, Lk, True)
        out.append({"B": B, "Hq": Hq, "Hkv": Hkv, "Lq": Lq, "Lk": Lk,
                    "num_splits": S.attn_splitkv_num_splits(B, Hq, Hkv, Lq, Lk, D, D),
                    "attn_fwd_ms": round(ms_f, 4), "split_ms": round(ms_s, 4),
                    "split_tflops": round(flops / (ms_s * 1e-3) / 1e12, 1)})
        del q, k, v, o, lse, ws
    torch.cuda.empty_cache()
    return out


def bench_crossover(lengths, topk=96, n_cols=1000, steps=3, warmup=2):
    """Dense causal attention (attn_fwd) against the dynamic sparse path (attn_build_sparse_index
    then attn_fwd_blocksparse on the built lists) as the sequence grows, at B 1, Hq 32, Hkv 8,
    D 128, with the index budget of the 128K workload at every length (96 key blocks per query
    block, 1000 columns per head). Inputs: seeded device N(0, 1) in bf16."""
    import torch
    import sparse_attention_attn_amd as S
    from workloads import randn_bf16_device
    B, Hq, Hkv, D = 1, 32, 8, 128
    scale = D ** -0.5
    out = []
    for L in lengths:
        q = randn_bf16_device((B, L, Hq, D), 7000 + L)
        k = randn_bf16_device((B, L, Hkv, D), 7001 + L)
        v = randn_bf16_device((B, L, Hkv, D), 7002 + L)
        o = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device="cuda:0")
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda:0")
        ms_dense, _ = time_steps(lambda: S.attn_fwd(q, k, v, o, lse, causal=True, scale=scale),
                                 steps, warmup)
        nb, nc = S.attn_sparse_index_sizes(B, Hq, L, topk, n_cols)
        nqb = -(-L // 64)
        outs = (torch.empty(B * Hq * nqb + 1, dtype=torch.int32, device="cuda:0"),
                torch.empty(max(nb, 1), dtype=torch.int32, device="cuda:0"),
                torch.empty(B * Hq + 1, dtype=torch.int32, device="cuda:0"),
                torch.empty(max(nc, 1), dtype=torch.int32, device="cuda:0"))
        ws = torch.empty(S.attn_sparse_index_workspace_bytes(B, Hq, Hkv, L, D), dtype=torch.uint8,
                         device="cuda:0")
        build = lambda: S.attn_build_sparse_index(q, k, topk, n_cols, scale=scale, outputs=outs,
                                                  workspace=ws)
        ms_build, _ = time_steps(build, steps, warmup)
        lists = build()
        ms_sparse, _ = time_steps(lambda: S.attn_fwd_blocksparse(q, k, v, o, *lists, lse=lse,
                                                                 causal=True, scale=scale),
                                  steps, warmup)
        torch.cuda.synchronize()
        hl = [t.cpu().numpy() for t in lists]
        pairs = blocksparse_pairs(hl, B, Hq, L)
        dense_pairs = B * Hq * dense_causal_pairs(L, L, True)
        rec = {"L": L, "dense_ms": round(ms_dense, 4), "build_ms": round(ms_build, 4),
               "sparse_ms": round(ms_sparse, 4),
               "build_plus_sparse_ms": round(ms_build + ms_sparse, 4),
               "density_vs_causal": round(pairs / dense_pairs, 4),
               "speedup_vs_dense": round(ms_dense / (ms_build + ms_sparse), 3)}
        out.append(rec)
        log(f"  crossover {rec}")
        del q, k, v, o, lse, outs, ws, lists
        torch.cuda.empty_cache()
    return out


def bench_entry_memory():
    """Peak device memory of the other entry points at long context, above the op's inputs and
    outputs, with the workspaces the binding allocates for the call counted (torch's peak
    counter; the library itself allocates nothing): block-sparse, vertical-slash and both index
    builders at the 128K workloads' shape, the GQA decode and the MLA decode at 131072 keys."""
    import numpy as np
    import torch
    import sparse_attention_attn_amd as S
    from workloads import make_blocksparse_lists, make_vslash_lists, randn_bf16_device
    dev = "cuda:0"
    out = []

    def measure(name, tensors, fn, note):
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        fn()
        torch.cuda.synchronize()
        extra = torch.cuda.max_memory_allocated() - base
        io = sum(t.numel() * t.element_size() for t in tensors)
        rec = {"entry": name, "inputs_outputs_bytes": int(io), "extra_bytes": int(extra),
               "note": note}
        out.append(rec)
        log(f"  entry memory {rec}")

    B, Hq, Hkv, L, D = 1, 32, 8, 131072, 128
    q = randn_bf16_device((B, L, Hq, D), 8100)
    k = randn_bf16_device((B, L, Hkv, D), 8101)
    v = randn_bf16_device((B, L, Hkv, D), 8102)
    o = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    bl = [torch.from_numpy(np.ascontiguousarray(x)).to(dev)
          for x in make_blocksparse_lists(B, Hq, L, L, 5003)]
    measure("attn_fwd_blocksparse", [q, k, v, o, lse] + bl,
            lambda: S.attn_fwd_blocksparse(q, k, v, o, *bl, lse=lse, causal=True),
            "B 1, Hq 32, Hkv 8, D 128, L 131072; index lists counted as inputs")
    sp, si, cp, ci = [torch.from_numpy(np.ascontiguousarray(x)).to(dev)
                      for x in make_vslash_lists(B, Hq, L, 6003)]
    nqb = -(-L // 64)
    bp0 = torch.zeros(B * Hq * nqb + 1, dtype=torch.int32, device=dev)
    bi0 = torch.zeros(1, dtype=torch.int32, device=dev)
    measure("attn_fwd_vertical_slash", [q, k, v, o, lse, sp, si, cp, ci, bp0, bi0],
            lambda: S.attn_fwd_vertical_slash(q, k, v, o, bp0, bi0, cp, ci, sp, si, lse=lse),
            "same shape; extra = the two per-head bitmaps of its workspace")
    measure("attn_build_sparse_index", [q, k],
            lambda: S.attn_build_sparse_index(q, k, 96, 1000),
            "same shape, 96 blocks per query block, 1000 columns; extra = output lists + "
            "workspace")
    measure("attn_build_vslash_index", [q, k],
            lambda: S.attn_build_vslash_index(q, k, 1000, 1088),
            "same shape, 1000 columns, 1088 slash lines; extra = output lists + workspace")
    del q, k, v, o, lse, bl, sp, si, cp, ci, bp0, bi0
    torch.cuda.empty_cache()
    for (Bd, Hqd, Hkvd, Dqk, Dv, name) in ((16, 32, 8, 128, 128, "GQA"), (8, 16, 1, 576, 512, "MLA")):
        Lk = 131072
        qd = randn_bf16_device((Bd, 1, Hqd, Dqk), 8200)
        kd = randn_bf16_device((Bd, Lk, Hkvd, Dqk), 8201)
        vd = kd[..., :Dv] if Dqk != Dv else randn_bf16_device((Bd, Lk, Hkvd, Dv), 8202)
        od = torch.empty((Bd, 1, Hqd, Dv), dtype=torch.bfloat16, device=dev)
        ld = torch.empty((Bd, Hqd, 1), dtype=torch.float32, device=dev)
        ins = [qd, kd, od, ld] + ([] if Dqk != Dv else [vd])
        measure(f"attn_fwd_decode ({name})", ins,
                lambda: S.attn_fwd_decode(qd, kd, vd, od, ld),
                f"B {Bd}, Hq {Hqd}, Hkv {Hkvd}, Dqk {Dqk}, Dv {Dv}, 131072 keys; extra = the "
                "split-KV partials workspace")
        measure(f"attn_fwd_decode_noalloc ({name})", ins,
                lambda: S.attn_fwd_decode_noalloc(qd, kd, vd, od, ld),
                "same shape; partials in the library's static scratch array")
        del qd, kd, vd, od, ld
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


def oracle_timings(threads_all, budget_s=15.0):
    """The fp64 oracle, as it stands, timed on the other workloads (beside the headline entry of
    cpu_baseline): the tiny causal prefill, the GQA decode and the MLA decode in full, each on
    all host threads and on one thread; the 128K block-sparse prefill on its 4096 sampled query
    rows (rows 0-63, the last 64 and 3968 seeded rows) of all 32 heads, each query block's rows
    over that block's listed keys, with a x32 linear extrapolation to all 131072 rows labelled
    as such. Rates use the GPU rows' algorithmic counts: TFLOP/s of visible pairs for prefill,
    GB/s of K/V (+ Q, O, LSE) bytes for decode."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import attention as A
    from workloads import WORKLOADS, make_blocksparse_lists, make_qkv, sampled_rows
    f64 = lambda t: t.float().numpy().astype(np.float64)
    out = []

    def run_full(w, threads):
        q, k, v = make_qkv(w)
        qf, kf = f64(q), f64(k)
        vf = A.mla_value_view(kf, w.Dv) if w.mla else f64(v)
        with threadpool_limits(limits=threads):
            t0 = time.perf_counter()
            A.attention(qf, kf, vf, A.effective_scale(w.scale), w.causal)
            el = time.perf_counter() - t0
        rec = {"workload": w.name, "threads": threads, "seconds": round(el, 3),
               "sample": "whole workload"}
        if w.kind == "prefill":
            fl = 2 * (w.Dqk + w.Dv) * w.B * w.Hq * dense_causal_pairs(w.Lq, w.Lk, w.causal)
            rec.update({"value": fl / el / 1e12, "unit": "TFLOP/s"})
        else:
            nbytes = k.numel() * 2 + (0 if w.mla else v.numel() * 2) + q.numel() * 2 + \
                w.B * w.Lq * w.Hq * w.Dv * 2 + w.B * w.Hq * w.Lq * 4
            rec.update({"value": nbytes / el / 1e9, "unit": "GB/s"})
        return rec

    for name in ("tiny_causal", "gqa_decode_4k", "mla_decode_64k"):
        for th in sorted({threads_all, 1}, reverse=True):
            out.append(run_full(WORKLOADS[name], th))
            log(f"  oracle {out[-1]}")

    w = WORKLOADS["blocksparse_128k"]
    q, k, v = make_qkv(w)
    bp, bi, cp, ci = make_blocksparse_lists(w.B, w.Hq, w.Lq, w.Lk, 1000 * w.index + 3)
    rows = sampled_rows(w.Lq, 4096, 1000 * w.index + 4, edge=64)
    nqb = -(-w.Lq // 64)
    sc = A.effective_scale(w.scale)
    qbs = rows // 64
    pairs = 0
    el = 0.0
    heads = 0
    for h in range(w.Hq):
        if el >= budget_s:
            break
        heads += 1
        kh = f64(k[0, :, h // (w.Hq // w.Hkv)])
        vh = f64(v[0, :, h // (w.Hq // w.Hkv)])
        qh = f64(q[0, rows, h])
        cols = ci[cp[h]:cp[h + 1]]
        t0 = time.perf_counter()
        for qb in np.unique(qbs):
            sel = qbs == qb
            keys = A.blocksparse_keys(bi[bp[h * nqb + qb]:bp[h * nqb + qb + 1]], cols, w.Lk)
            A.attention_rows_over_keys(qh[sel], rows[sel], kh, vh, sc, keys, w.Lq, w.Lk, True)
            pairs += int(np.sum(np.searchsorted(keys, rows[sel], side="right")))
        el += time.perf_counter() - t0
    fl = 2 * (w.Dqk + w.Dv) * pairs
    out.append({"workload": w.name, "threads": threads_all, "seconds": round(el, 3),
                "value": fl / el / 1e12, "unit": "TFLOP/s",
                "sample": f"{len(rows)} of {w.Lq} query rows x {heads} of {w.Hq} heads, over "
                          f"each query block's listed keys ({pairs} visible pairs)",
                "extrapolated_seconds_whole_workload": round(
                    el * (w.Lq / len(rows)) * (w.Hq / heads), 1),
                "extrapolation": f"linear: x{w.Lq // len(rows)} rows, x{w.Hq / heads:g} heads"})
    log(f"  oracle {out[-1]}")
    return out


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
    ap.add_argument("--no-dynamic", action="store_true",
                    help="block-sparse and vertical-slash: skip the built-list (index builder) "
                         "measurements, so a profile of the run holds the static-list launches only")
    ap.add_argument("--no-crossover", action="store_true",
                    help="skip the dense vs dynamic sparse sweep over sequence length")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the bf16 GEMM / device copy measurement of achievable peaks")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-oracle-others", action="store_true",
                    help="time the oracle on the headline workload only")
    ap.add_argument("--min-warmup-ms", type=float, default=300.0,
                    help="keep warming up (untimed) until this much wall time has passed")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration)")
    args = ap.parse_args()
    global MIN_WARMUP_S
    MIN_WARMUP_S = max(0.0, args.min_warmup_ms) / 1000.0

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
            res[name] = bench_blocksparse(w, max(3, args.steps // 4), min(args.warmup, 2),
                                          dynamic=not args.no_dynamic)
        elif w.kind == "vslash":
            res[name] = bench_vslash(w, max(3, args.steps // 4), min(args.warmup, 2),
                                     dynamic=not args.no_dynamic)
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
            "warmup_steps_run": r.get("warmup_steps_run"),
            "min_warmup_ms": args.min_warmup_ms,
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
                                                          ach["achievable_mfma_tflops"], 4)
    wl = {}
    for name, r in res.items():
        pct = {kk: r[kk] for kk in ("ms_p10", "ms_p50", "ms_p90", "warmup_steps_run") if kk in r}
        if "gbs" in r:
            wl[name] = {"value": round(r["gbs"], 1), "unit": "GB/s", "ms": round(r["ms"], 4),
                        **pct, "frac_of_hbm_peak": round(r["gbs"] / HBM_PEAK_GBS, 4),
                        "num_splits": r["num_splits"], "bytes": r["bytes"]}
            if ach:
                wl[name]["frac_of_achievable"] = round(r["gbs"] / ach["achievable_hbm_read_gbs"], 4)
            fl = r.get("read_floor")
            if fl is not None:
                wl[name]["read_floor"] = fl
                if "ms" in fl:
                    wl[name]["frac_of_read_floor"] = round(fl["ms"] / r["ms"], 4)
        else:
            wl[name] = {"value": round(r["tflops"], 3), "unit": "TFLOP/s", "ms": round(r["ms"], 4),
                        **pct, "frac_of_mfma_peak": round(r["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
                        "flops": r["flops"]}
            if ach:
                wl[name]["frac_of_achievable"] = round(r["tflops"] / ach["achievable_mfma_tflops"],
                                                       4)
            if "density_vs_causal" in r:
                wl[name]["density_vs_causal"] = round(r["density_vs_causal"], 4)
            if "dynamic" in r:
                wl[name]["dynamic_index"] = r["dynamic"]
            if "dynamic_structured" in r:
                wl[name]["dynamic_index_structured"] = r["dynamic_structured"]
        if name in SPARSE_WORKLOADS:
            # L2-miss traffic (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated, taken on the
            # current kernel source) over this run's step time, against the read ceiling
            sparse_hash = kernel_source_hash(SPARSE_SOURCES)
            tb = load_traffic(name, sparse_hash)
            entry = {"bytes_per_launch": tb, "kernel_source_sha256_16": sparse_hash}
            if tb is not None:
                entry["rate_gbs"] = round(tb / (r["ms"] * 1e-3) / 1e9, 1)
                ceil = (ach or {}).get("read_ceilings", {}).get("infinity_cache_tile_gather_read_gbs")
                if ceil:
                    entry["read_ceiling_gbs"] = ceil
                    entry["frac_of_read_ceiling"] = round(entry["rate_gbs"] / ceil, 4)
            wl[name]["l2_miss_traffic"] = entry
    out["workloads"] = wl
    if not args.no_etap_grid and args.only is None:
        log("FlashMLA-ETAP decode grid ...")
        out["etap_grid"] = {"unit": "one attn_fwd_decode per step; TFLOP/s = 2*(576+512) per "
                                    "visible (query, key) pair; GB/s = latent cache + Q + O + LSE",
                            "points": bench_etap_grid(max(5, args.steps // 2), 3)}
    if not args.no_crossover and args.only is None:
        log("prefill shapes ...")
        out["prefill_sweep"] = {
            "op": "causal GQA prefill, D 128; TFLOP/s over the visible (query, key) pairs",
            "points": bench_prefill_sweep([(1, 8, 2, 2048), (1, 8, 2, 8192), (1, 8, 2, 32768),
                                           (1, 32, 8, 2048), (1, 32, 8, 4096), (4, 32, 8, 4096),
                                           (1, 64, 8, 16384), (2, 32, 8, 32768)])}
    if not args.no_crossover and args.only is None:
        log("chunked prefill ...")
        out["chunked_prefill"] = {
            "op": "causal GQA prefill of a query chunk against a longer cache, D 128",
            "points": bench_chunked_prefill([(1, 32, 8, 512, 32768), (1, 32, 8, 1024, 16384),
                                             (4, 32, 8, 256, 16384)])}
    if not args.no_memory and args.only is None:
        log("peak memory at long sequence lengths ...")
        out["memory"] = {"op": "causal prefill B 1, Hq 32, Hkv 8, D 128",
                         "points": bench_memory([4096, 8192, 16384, 32768, 65536, 131072],
                                                eager_max=16384)}
    if not args.no_crossover and args.only is None:
        log("dense vs dynamic sparse crossover ...")
        out["sparse_crossover"] = {
            "op": "causal prefill B 1, Hq 32, Hkv 8, D 128: attn_fwd against "
                  "attn_build_sparse_index + attn_fwd_blocksparse (96 blocks per query block, "
                  "1000 columns per head at every length)",
            "points": bench_crossover([4096, 8192, 16384, 32768, 65536, 131072])}
    if not args.no_memory and args.only is None:
        log("peak memory of the other entry points ...")
        out["entry_memory"] = bench_entry_memory()
    if not args.no_cpu_baseline and HEADLINE in res:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(head, args.cpu_seconds)
        if not args.no_oracle_others:
            log("oracle on the other workloads ...")
            out["cpu_baseline"]["other_workloads"] = oracle_timings(out["cpu_baseline"]["cores"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

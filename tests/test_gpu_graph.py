"""HIP-graph capture of the library's calls (torch.cuda.graph over the C-ABI launches): the
decode step (attn_fwd_decode: split-KV + combine), the prefill, the block-sparse and
vertical-slash forwards, and the two dynamic pipelines (index builder, then the sparse forward
over the lists it wrote, in one graph). Each is captured once and replayed several times with
the program's own eager work and synchronizations between the replays; every replay must
equal the eager result bitwise (the kernels are deterministic). No library call records a
memset or allocates: buffers and workspaces are passed in."""

import pytest

from tests.helpers import say
from workloads import randn_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _replays_match(run, outs, label):
    import torch
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for i in range(4):
        for t in outs:
            t.fill_(0)                       # eager work between replays
        noise = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"{label}: replay {i} differs from the eager result"
        del noise


@pytest.mark.parametrize("shape", [(16, 32, 8, 1, 4096, 128, 128), (4, 16, 1, 2, 3000, 576, 512),
                                   (128, 16, 4, 2, 300, 128, 128),
                                   (1, 16, 4, 384, 3000, 128, 128)],
                         ids=["gqa", "mla", "one_split_direct", "chunked_prefill"])
def test_decode_graph_replays_equal_eager(shape):
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, Lq, Lk, Dqk, Dv = shape
    say(f"graph decode {shape}")
    q = randn_bf16((B, Lq, Hq, Dqk), 8950).to(DEV)
    k = randn_bf16((B, Lk, Hkv, Dqk), 8951).to(DEV)
    v = k[..., :Dv] if Dqk != Dv else randn_bf16((B, Lk, Hkv, Dv), 8952).to(DEV)
    o = torch.empty((B, Lq, Hq, Dv), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(256, S.attn_decode_workspace_bytes(B, Hq, Hkv, Lq, Lk, Dqk, Dv)),
                     dtype=torch.uint8, device=DEV)
    if Lk < 512:
        assert S.attn_splitkv_num_splits(B, Hq, Hkv, Lq, Lk, Dqk, Dv) == 1
    _replays_match(lambda: S.attn_fwd_decode(q, k, v, o, lse, causal=Lq > 1, workspace=ws),
                   [o, lse], f"decode {shape}")


def test_prefill_graph_replays_equal_eager():
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, L, D = 1, 8, 2, 2048, 128
    say("graph prefill")
    q = randn_bf16((B, L, Hq, D), 8960).to(DEV)
    k = randn_bf16((B, L, Hkv, D), 8961).to(DEV)
    v = randn_bf16((B, L, Hkv, D), 8962).to(DEV)
    o = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    _replays_match(lambda: S.attn_fwd(q, k, v, o, lse, causal=True), [o, lse], "prefill")


def _sparse_inputs(B, Hq, Hkv, L, D, seed):
    import torch
    q = randn_bf16((B, L, Hq, D), seed).to(DEV)
    k = randn_bf16((B, L, Hkv, D), seed + 1).to(DEV)
    v = randn_bf16((B, L, Hkv, D), seed + 2).to(DEV)
    o = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    return q, k, v, o, lse


def test_blocksparse_graph_replays_equal_eager():
    import torch
    import sparse_attention_attn_amd as S
    from workloads import make_blocksparse_lists
    B, Hq, Hkv, L, D = 1, 8, 2, 3000, 128
    say("graph block-sparse")
    q, k, v, o, lse = _sparse_inputs(B, Hq, Hkv, L, D, 8970)
    lists = [torch.as_tensor(x).to(DEV)
             for x in make_blocksparse_lists(B, Hq, L, L, 8973, local_blocks=8, p_extra=0.1,
                                             n_cols=40)]
    _replays_match(lambda: S.attn_fwd_blocksparse(q, k, v, o, *lists, lse=lse, causal=True),
                   [o, lse], "block-sparse")


def test_vslash_graph_replays_equal_eager():
    import torch
    import sparse_attention_attn_amd as S
    from workloads import make_vslash_lists
    B, Hq, Hkv, L, D = 1, 8, 2, 3000, 128
    say("graph vertical-slash")
    q, k, v, o, lse = _sparse_inputs(B, Hq, Hkv, L, D, 8980)
    sp, si, cp, ci = [torch.as_tensor(x).to(DEV)
                      for x in make_vslash_lists(B, Hq, L, 8983, band=200, n_far=12, n_cols=50)]
    nqb = -(-L // 64)
    bp = torch.zeros(B * Hq * nqb + 1, dtype=torch.int32, device=DEV)
    bi = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(256, S.attn_vertical_slash_workspace_bytes(B, Hq, L)), dtype=torch.uint8,
                     device=DEV)
    _replays_match(lambda: S.attn_fwd_vertical_slash(q, k, v, o, bp, bi, cp, ci, sp, si, lse=lse,
                                                     causal=True, workspace=ws),
                   [o, lse], "vertical-slash")


def test_dynamic_blocksparse_pipeline_graph_replays_equal_eager():
    """attn_build_sparse_index then attn_fwd_blocksparse over its lists, captured together."""
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, L, D, topk, ncols = 1, 8, 2, 4096, 128, 12, 64
    say("graph dynamic block-sparse pipeline")
    q, k, v, o, lse = _sparse_inputs(B, Hq, Hkv, L, D, 8990)
    nb, nc = S.attn_sparse_index_sizes(B, Hq, L, topk, ncols)
    nqb = -(-L // 64)
    mk = lambda n: torch.empty(max(int(n), 1), dtype=torch.int32, device=DEV)
    outs = (mk(B * Hq * nqb + 1), mk(nb), mk(B * Hq + 1), mk(nc))
    ws = torch.empty(max(256, S.attn_sparse_index_workspace_bytes(B, Hq, Hkv, L, D)),
                     dtype=torch.uint8, device=DEV)

    def run():
        lists = S.attn_build_sparse_index(q, k, topk, ncols, outputs=outs, workspace=ws)
        S.attn_fwd_blocksparse(q, k, v, o, *lists, lse=lse, causal=True)

    _replays_match(run, [o, lse, *outs], "dynamic block-sparse")


def test_dynamic_vslash_pipeline_graph_replays_equal_eager():
    """attn_build_vslash_index then attn_fwd_vertical_slash over its lists, captured together."""
    import torch
    import sparse_attention_attn_amd as S
    B, Hq, Hkv, L, D, ncols, nslash = 1, 8, 2, 4096, 128, 64, 96
    say("graph dynamic vertical-slash pipeline")
    q, k, v, o, lse = _sparse_inputs(B, Hq, Hkv, L, D, 9000)
    mk = lambda n: torch.empty(max(int(n), 1), dtype=torch.int32, device=DEV)
    outs = (mk(B * Hq + 1), mk(B * Hq * ncols), mk(B * Hq + 1), mk(B * Hq * nslash))
    ws = torch.empty(max(256, S.attn_sparse_index_workspace_bytes(B, Hq, Hkv, L, D)),
                     dtype=torch.uint8, device=DEV)
    vws = torch.empty(max(256, S.attn_vertical_slash_workspace_bytes(B, Hq, L)), dtype=torch.uint8,
                      device=DEV)
    nqb = -(-L // 64)
    bp = torch.zeros(B * Hq * nqb + 1, dtype=torch.int32, device=DEV)
    bi = torch.zeros(1, dtype=torch.int32, device=DEV)

    def run():
        cp, ci, sp, si = S.attn_build_vslash_index(q, k, ncols, nslash, outputs=outs, workspace=ws)
        S.attn_fwd_vertical_slash(q, k, v, o, bp, bi, cp, ci, sp, si, lse=lse, causal=True,
                                  workspace=vws)

    _replays_match(run, [o, lse, *outs], "dynamic vertical-slash")

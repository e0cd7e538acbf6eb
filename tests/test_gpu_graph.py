"""HIP-graph capture of the library's calls (torch.cuda.graph over the C-ABI launches): the
decode step (attn_fwd_decode: split-KV + combine) and the prefill, each captured once and
replayed several times with the program's own eager work and synchronizations between the
replays; every replay must equal the eager result bitwise (the kernels are deterministic)."""

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
                                   (2, 16, 4, 2, 300, 128, 128)],
                         ids=["gqa", "mla", "one_split_direct"])
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

"""The binding launches on the caller's stream: torch's current stream unless one is passed.
Checked on the stream handle the binding resolves and on results computed on a side stream
while the default stream is kept busy."""

import pytest

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_binding_resolves_the_current_stream():
    import torch
    from sparse_attention_attn_amd import _lib
    dev = torch.device(DEV)
    assert _lib._stream(None, dev) == torch.cuda.current_stream(dev).cuda_stream
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        assert _lib._stream(None, dev) == s.cuda_stream
    assert _lib._stream(None, dev) == torch.cuda.current_stream(dev).cuda_stream
    assert _lib._stream(s.cuda_stream, dev) == s.cuda_stream


def test_side_stream_results_match_default_stream():
    """attn_fwd and attn_fwd_decode on a side stream give the default stream's results
    bit for bit; the default stream is busy with unrelated work meanwhile."""
    import torch
    import sparse_attention_attn_amd as S
    from workloads import randn_bf16_device
    q = randn_bf16_device((2, 300, 8, 128), 9980)
    k = randn_bf16_device((2, 300, 2, 128), 9981)
    v = randn_bf16_device((2, 300, 2, 128), 9982)
    o_ref = torch.empty_like(q)
    l_ref = torch.empty((2, 8, 300), dtype=torch.float32, device=DEV)
    S.attn_fwd(q, k, v, o_ref, l_ref, causal=True)
    qd = q[:, -1:].contiguous()
    od_ref = torch.empty_like(qd)
    ld_ref = torch.empty((2, 8, 1), dtype=torch.float32, device=DEV)
    S.attn_fwd_decode(qd, k, v, od_ref, ld_ref, causal=True)
    torch.cuda.synchronize()
    busy = torch.randn((4096, 4096), device=DEV)
    s = torch.cuda.Stream(device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty_like(l_ref)
    od = torch.empty_like(qd)
    ld = torch.empty_like(ld_ref)
    s.wait_stream(torch.cuda.current_stream())
    for _ in range(4):
        busy = busy @ busy.T * 1e-3   # default-stream work
    with torch.cuda.stream(s):
        S.attn_fwd(q, k, v, o, lse, causal=True)
        S.attn_fwd_decode(qd, k, v, od, ld, causal=True)
    s.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    assert torch.equal(od, od_ref) and torch.equal(ld, ld_ref)
    torch.cuda.synchronize()

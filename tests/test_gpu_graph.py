"""The entry points launch kernels only (no allocation, memset or
synchronization), so a caller can capture them in a HIP graph.  Each call is
captured once and replayed several times, with unrelated eager work and
synchronizations between the replays; every replay must equal the eager call
bit for bit (the kernels are deterministic)."""
import math

import pytest
import torch

from long_context_attention_jl_amd import inputs
from long_context_attention_jl_amd import jetlong as jl

from _parity import say

pytestmark = pytest.mark.gpu

PARAMS = dict(w_pretrained=256, w_local=64, rope_base=1e4, softmax_scale=1.0 / math.sqrt(128))


def _replays_equal(fn, outs, n=3):
    """fn() writes into outs; capture it, replay n times, compare with eager."""
    fn()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    for t in outs:
        t.fill_(float("nan")) if t.is_floating_point() else t.zero_()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream, as torch's docs advise
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    noise = torch.randn(1024, 1024, device="cuda")
    for r in range(n):
        for t in outs:
            t.fill_(float("nan")) if t.is_floating_point() else t.zero_()
        g.replay()
        noise = noise @ noise.t() / 1024.0  # unrelated eager work between replays
        torch.cuda.synchronize()
        for a, b in zip(outs, want):
            assert torch.equal(a, b), "replay %d differs from the eager call" % r
    say("graph replays equal eager:", n)


def test_graph_decode():
    B, S, Hq, Hkv, d = 2, 3000, 8, 2, 128
    q, kc, vc = inputs.decode_inputs(B, S, Hq, Hkv, d, seed=41)
    q, kc, vc = q.cuda(), kc.cuda(), vc.cuda()
    sl = torch.tensor([3000, 1777], dtype=torch.int32, device="cuda")
    ws = torch.empty(jl.decode_workspace_bytes(B, S, Hq, Hkv, d, q.dtype), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    _replays_equal(lambda: jl.bifocal_decode(q, kc, vc, sl, max_seqlen_k=S, workspace=ws, out=o,
                                             lse_out=lse, **PARAMS), [o, lse])


def test_graph_prefill():
    T, Hq, Hkv, d = 1500, 4, 2, 128
    q, k, v = inputs.prefill_inputs(T, Hq, Hkv, d, seed=42)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    ws = torch.empty(jl.prefill_workspace_bytes(T, 1, Hq, Hkv, d, q.dtype), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
    _replays_equal(lambda: jl.bifocal_prefill(q, k, v, workspace=ws, out=o, lse_out=lse, **PARAMS),
                   [o, lse])


def test_graph_chunk():
    chunks, lens, S = [300, 1], [2500, 900], 2500
    q, kc, vc, cu = inputs.chunk_inputs(chunks, lens, S, 8, 2, 128, seed=43)
    q, kc, vc = q.cuda(), kc.cuda(), vc.cuda()
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda")
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ws = torch.empty(jl.prefill_chunk_workspace_bytes(sum(chunks), len(lens), S, 8, 2, 128),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((8, sum(chunks)), dtype=torch.float32, device="cuda")
    _replays_equal(lambda: jl.bifocal_prefill_chunk(q, kc, vc, sl, cu_seqlens_q=cu_t,
                                                    max_seqlen_q=max(chunks), max_seqlen_k=S,
                                                    workspace=ws, out=o, lse_out=lse, **PARAMS),
                   [o, lse])

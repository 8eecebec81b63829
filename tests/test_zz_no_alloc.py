"""jl_bifocal_decode_noalloc (the library's static scratch, no workspace)
against jl_bifocal_decode through the C ABI: the same kernels on the same
inputs, so the outputs must be identical, on two calls in a row with the
second smaller (the scratch keeps the first call's partials, and its merge
counters must be back at zero), and both within the oracle's bars."""
import math

import pytest
import torch

import oracle
from long_context_attention_jl_amd import inputs
from long_context_attention_jl_amd import jetlong as jl
from long_context_attention_jl_amd.inputs import Params

from _parity import check_decode, say

pytestmark = pytest.mark.gpu


def _both(q, kc, vc, lens, p, S):
    B, Hq, d = q.shape
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o1 = torch.full((B, Hq, d), float("nan"), dtype=q.dtype, device="cuda")
    l1 = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    kw = dict(w_pretrained=p.w_pretrained, w_local=p.w_local, rope_base=p.rope_base,
              softmax_scale=p.softmax_scale, max_seqlen_k=S)
    jl.bifocal_decode_noalloc(qd, kd, vd, sl, o1, l1, **kw)
    o0, l0 = jl.bifocal_decode(qd, kd, vd, sl, **kw)
    torch.cuda.synchronize()
    return o1, l1, o0, l0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_decode_matches_workspace_decode_twice(dtype):
    p = Params(4096, 700, 1e6, 1.0 / math.sqrt(128))
    cases = [(2, 20000, 32, 8, [20000, 9001]),  # several bins of chunks per sequence
             (1, 3000, 8, 2, [2999])]           # then a smaller call on the same scratch
    for B, S, Hq, Hkv, lens in cases:
        say("noalloc decode", dtype, B, S, Hq, Hkv, lens)
        q, kc, vc = inputs.decode_inputs(B, S, Hq, Hkv, 128, seed=S + B, dtype=dtype)
        o1, l1, o0, l0 = _both(q, kc, vc, lens, p, S)
        assert torch.equal(o1, o0) and torch.equal(l1, l0), "noalloc differs from jl_bifocal_decode"
        o_ref, l_ref = oracle.decode(q, kc, vc, lens, w_pretrained=p.w_pretrained,
                                     w_local=p.w_local, rope_base=p.rope_base,
                                     softmax_scale=p.softmax_scale)
        check_decode(o1, l1, o_ref, l_ref, dtype, "noalloc B=%d S=%d" % (B, S))

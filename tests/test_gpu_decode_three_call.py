"""GPU parity of the pages' unfused generation step (jl_bifocal_decode_three_call):
the cache's keys turned to remapped RoPE, calls B (every key remapped), A
(local keys, standard) and C (local keys, remapped) and the LogSumExp merge
must equal the direct bifocal decode the oracle computes, within the bf16
bars, and agree with the fused decode."""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_attention_jl_amd import inputs
from long_context_attention_jl_amd import jetlong as jl
from long_context_attention_jl_amd.inputs import Params

from _parity import check_decode, say

pytestmark = pytest.mark.gpu


def _kw(p):
    return dict(w_pretrained=p.w_pretrained, w_local=p.w_local, rope_base=p.rope_base,
                softmax_scale=p.softmax_scale)


def _ref(q, kc, vc, lens, p, bifocal=True):
    return oracle.decode(q, kc, vc, lens, bifocal=bifocal, **_kw(p))


def test_three_call_decode_128k():
    """L = 131072 (G = 4): against the oracle, with discrimination, and against
    the fused decode; the cache is left unchanged."""
    c = inputs.decode_128k()
    kc, vc = c.k_cache.cuda(), c.v_cache.cuda()
    before = kc.clone()
    o, lse = jl.bifocal_decode_three_call(c.q.cuda(), kc, vc, c.seqlens, **_kw(c.params))
    torch.cuda.synchronize()
    assert torch.equal(kc, before), "the cache must never be rewritten"
    o_ref, l_ref = _ref(c.q, c.k_cache, c.v_cache, c.seqlens, c.params)
    o_pl, _ = _ref(c.q, c.k_cache, c.v_cache, c.seqlens, c.params, bifocal=False)
    check_decode(o, lse, o_ref, l_ref, torch.bfloat16, "three-call decode 128K", o_plain=o_pl)
    o_f, l_f = jl.bifocal_decode(c.q.cuda(), kc, vc, c.seqlens, **_kw(c.params))
    torch.cuda.synchronize()
    dO = (o_f.float() - o.float()).abs().max().item()
    dL = (l_f - lse).abs().max().item()
    say("fused vs three-call decode: max|dO|=%.3g max|dLSE|=%.3g" % (dO, dL))
    assert dO <= 2e-2 and dL <= 1e-3


def test_three_call_decode_16_steps_across_g_switch():
    queries, kc_h, vc_h, lens, p = inputs.decode_16step_cache()
    kc, vc = kc_h.cuda(), vc_h.cuda()
    for step, (q, L) in enumerate(zip(queries, lens)):
        o, lse = jl.bifocal_decode_three_call(q.cuda(), kc, vc, [L], max_seqlen_k=L, **_kw(p))
        torch.cuda.synchronize()
        o_ref, l_ref = _ref(q, kc_h, vc_h, [L], p)
        check_decode(o, lse, o_ref, l_ref, torch.bfloat16, "three-call step %d L=%d" % (step, L))


@pytest.mark.parametrize("d,Hq,Hkv", [(128, 8, 2), (64, 16, 1), (128, 24, 12)])
def test_three_call_decode_batched_mixed_lengths(d, Hq, Hkv):
    """Three sequences of 700, 1 and 333 keys in a cache of 900 rows per
    sequence (so the remapped copy's rows differ from the cache's)."""
    B, S = 3, 900
    q, kc, vc = inputs.decode_inputs(B, S, Hq, Hkv, d, seed=d + Hq + 11)
    lens = [700, 1, 333]
    p = Params(100, 50, 1e4, 1.0 / math.sqrt(d))
    o, lse = jl.bifocal_decode_three_call(q.cuda(), kc.cuda(), vc.cuda(), lens, max_seqlen_k=700,
                                          **_kw(p))
    torch.cuda.synchronize()
    o_ref, l_ref = _ref(q, kc, vc, lens, p)
    check_decode(o, lse, o_ref, l_ref, torch.bfloat16, "three-call batched d=%d" % d)


@pytest.mark.parametrize("label,p", [
    ("w_local0", Params(64, 0, 1e4, 0.1)),        # A and C empty: B alone
    ("w_local_all", Params(64, 4000, 1e4, 0.1)),  # every key local: B == C, A alone
    ("G1", Params(5000, 100, 1e4, 0.1)),          # L <= w_pretrained: plain RoPE
    ("w_local1", Params(64, 1, 1e4, 0.1)),        # only the query's own key is local
])
def test_three_call_decode_degenerate(label, p):
    q, kc, vc = inputs.decode_inputs(2, 900, 8, 2, 128, seed=31)
    lens = [900, 517]
    o, lse = jl.bifocal_decode_three_call(q.cuda(), kc.cuda(), vc.cuda(), lens, **_kw(p))
    torch.cuda.synchronize()
    o_ref, l_ref = _ref(q, kc, vc, lens, p)
    check_decode(o, lse, o_ref, l_ref, torch.bfloat16, "three-call decode " + label)

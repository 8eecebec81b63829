"""GPU parity of the continuous-interpolation remote window (bifocal = 2: remote
position x / s with s = max(1, L / w_pretrained), the variant the pages compare
integer grouping against) for prefill, chunked prefill and decode (flat, paged
and fp8 caches), against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_attention_jl_amd import inputs
from long_context_attention_jl_amd import jetlong as jl
from long_context_attention_jl_amd.inputs import Params

from _parity import TOL_BF16_LSE, TOL_BF16_O, block_rows, check_decode, check_prefill, say

pytestmark = pytest.mark.gpu


def _kw(p, mode=2):
    return dict(w_pretrained=p.w_pretrained, w_local=p.w_local, rope_base=p.rope_base,
                softmax_scale=p.softmax_scale, bifocal=mode)


@pytest.mark.parametrize("T,Hq,Hkv,d,w_pre,w_local", [
    (700, 4, 2, 128, 200, 96),     # s = 3.5
    (3000, 4, 1, 128, 1024, 300),  # s = 2.93, rows >= 2048 in the main kernel
    (2600, 2, 2, 64, 700, 150),    # d = 64, s = 3.71
])
def test_interp_prefill_full(T, Hq, Hkv, d, w_pre, w_local):
    p = Params(w_pre, w_local, 1e4, 1.0 / math.sqrt(d))
    q, k, v = inputs.prefill_inputs(T, Hq, Hkv, d, seed=T + 7)
    say("interp prefill T=%d d=%d s=%.3f" % (T, d, T / w_pre))
    o, lse = jl.bifocal_prefill(q.cuda(), k.cuda(), v.cuda(), **_kw(p))
    torch.cuda.synchronize()
    rows = list(range(T))
    o_ref, l_ref = oracle.prefill(q, k, v, **_kw(p))
    o_int, _ = oracle.prefill(q, k, v, **_kw(p, 1))
    check_prefill(o, lse, o_ref, l_ref, rows, torch.bfloat16, "interp T=%d" % T, o_plain=o_int)


def test_interp_prefill_128k_every_workgroup():
    """The 128K layer with continuous interpolation: one row of every 256-row
    block plus the band-edge rows; every fourth row also under integer
    grouping, which the result must be told apart from."""
    c = inputs.qwen3_8b_128k()
    say("interp prefill", c.name)
    o, lse = jl.bifocal_prefill(c.q.cuda(), c.k.cuda(), c.v.cuda(), **_kw(c.params))
    torch.cuda.synchronize()
    rows = sorted(set(block_rows(c.T)) | {0, 5, 2046, 2047, 2048, 2049, 4097, 40001, 65537,
                                          100003, 131069, 131071})
    o_ref, l_ref = oracle.prefill(c.q, c.k, c.v, rows=rows, **_kw(c.params))
    o_int = o_ref.copy()
    o_int[::4], _ = oracle.prefill(c.q, c.k, c.v, rows=rows[::4], **_kw(c.params, 1))
    mask = np.zeros(len(rows), dtype=bool)
    mask[::4] = True
    check_prefill(o, lse, o_ref, l_ref, rows, torch.bfloat16, c.name + " interp",
                  o_plain=o_int, disc_rows=mask)


def test_interp_chunk():
    L, C = 2600, 900
    p = Params(1024, 256, 1e4, 1.0 / math.sqrt(128))
    q, kc, vc, _ = inputs.chunk_inputs([C], [L], L, 8, 2, 128, seed=55)
    say("interp chunk L=%d C=%d" % (L, C))
    o, lse = jl.bifocal_prefill_chunk(q.cuda(), kc.cuda(), vc.cuda(), [L], **_kw(p))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.prefill_chunk(q, kc, vc, [L], **_kw(p))
    check_prefill(o, lse, o_ref, l_ref, list(range(C)), torch.bfloat16, "interp chunk")


def _check_dec(o, lse, o_ref, l_ref, label):
    do = np.abs(o.float().cpu().double().numpy() - o_ref).max()
    dl = np.abs(lse.cpu().double().numpy() - l_ref).max()
    say("%s: max|dO|=%.3g max|dLSE|=%.3g" % (label, do, dl))
    assert do <= TOL_BF16_O and dl <= TOL_BF16_LSE, label


def test_interp_decode_batch_and_paged():
    B, S, Hq, Hkv, d = 3, 1500, 8, 2, 128
    lens = [1500, 1, 777]  # s = 5, 1, 2.59
    q, kc, vc = inputs.decode_inputs(B, S, Hq, Hkv, d, seed=61)
    p = Params(300, 100, 1e4, 1.0 / math.sqrt(d))
    say("interp decode lens=%s" % lens)
    o, lse = jl.bifocal_decode(q.cuda(), kc.cuda(), vc.cuda(), lens, max_seqlen_k=S, **_kw(p))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode(q, kc, vc, lens, **_kw(p))
    _check_dec(o, lse, o_ref, l_ref, "interp decode")
    page = 64
    npg = S // page + 1
    kp = torch.zeros((B * npg, page, Hkv, d), dtype=kc.dtype)
    vp = torch.zeros_like(kp)
    for b in range(B):
        for g in range(npg):
            r0, r1 = g * page, min((g + 1) * page, S)
            if r0 < r1:
                kp[b * npg + g, : r1 - r0] = kc[b, r0:r1]
                vp[b * npg + g, : r1 - r0] = vc[b, r0:r1]
    bt = torch.arange(B * npg, dtype=torch.int32).view(B, npg)
    o_p, l_p = jl.bifocal_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), bt.cuda(), lens,
                                       max_seqlen_k=S, **_kw(p))
    torch.cuda.synchronize()
    assert torch.equal(o, o_p) and torch.equal(lse, l_p)


def test_interp_decode_128k_bf16_and_fp8():
    c = inputs.decode_128k()
    say("interp decode 128K")
    o, lse = jl.bifocal_decode(c.q.cuda(), c.k_cache.cuda(), c.v_cache.cuda(), c.seqlens,
                               **_kw(c.params))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode(c.q, c.k_cache, c.v_cache, c.seqlens, **_kw(c.params))
    _check_dec(o, lse, o_ref, l_ref, "interp decode 128K")
    o_int, _ = oracle.decode(c.q, c.k_cache, c.v_cache, c.seqlens, **_kw(c.params, 1))
    err = np.linalg.norm(o.float().cpu().double().numpy() - o_ref)
    assert np.linalg.norm(o_ref - o_int) >= 10 * err, "interpolation indistinguishable from grouping"
    q, k8, v8, ks, vs, lens, p = inputs.decode_fp8_128k()
    o8, l8 = jl.bifocal_decode_fp8(q.cuda(), k8.cuda(), v8.cuda(), ks, vs, lens, **_kw(p))
    torch.cuda.synchronize()
    o8_ref, l8_ref = oracle.decode_fp8(q, k8, v8, ks.numpy(), vs.numpy(), lens, **_kw(p))
    _check_dec(o8, l8, o8_ref, l8_ref, "interp fp8 decode 128K")

"""GPU parity of the fp8 (OCP E4M3) cache: jl_kv_quantize_fp8 against the
oracle's quantizer (bit-exact codes), and jl_bifocal_decode_fp8 (flat and
paged) against the oracle's decode on the dequantized cache."""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_attention_jl_amd import inputs
from long_context_attention_jl_amd import jetlong as jl
from long_context_attention_jl_amd.inputs import Params

from _parity import TOL_BF16_LSE, TOL_BF16_O, say

pytestmark = pytest.mark.gpu


def _kw(p):
    return dict(w_pretrained=p.w_pretrained, w_local=p.w_local, rope_base=p.rope_base,
                softmax_scale=p.softmax_scale, bifocal=p.bifocal)


def _check(o, lse, o_ref, lse_ref, label):
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    do, dl = np.abs(og - o_ref).max(), np.abs(lg - lse_ref).max()
    say("%s: max|dO|=%.3g max|dLSE|=%.3g" % (label, do, dl))
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    assert do <= TOL_BF16_O and dl <= TOL_BF16_LSE, label


@pytest.mark.parametrize("ntok,H,d", [(333, 8, 128), (70, 2, 64), (1, 1, 8)])
def test_quantize_bit_exact(ntok, H, d):
    """Codes equal the oracle's (fp32 quotient, nearest-even, saturation) on
    values spanning subnormal codes, exact ties and saturation."""
    g = torch.Generator("cpu").manual_seed(ntok + H)
    x = (torch.randn(ntok, H, d, generator=g) * torch.logspace(-4, 1.5, d)).to(torch.bfloat16)
    scale = torch.rand(H, generator=g) * 0.05 + 0.002
    say("quantize ntok=%d H=%d d=%d" % (ntok, H, d))
    got = jl.kv_quantize_fp8(x.cuda(), scale.cuda())
    torch.cuda.synchronize()
    ref = oracle.e4m3_quant(x, scale.numpy())
    assert np.array_equal(got.cpu().numpy(), ref), "quantized codes differ"
    sat = np.abs(x.float().numpy() / scale.numpy()[None, :, None]) >= 448
    assert sat.any() and (ref[sat] & 0x7F == 0x7E).all()


@pytest.mark.parametrize("bifocal", [True, False])
def test_fp8_every_code_widens_exactly(bifocal):
    """A one-key decode returns the key's value row times the value scale
    exactly (the one probability is 1).  The value rows hold all 256 codes
    (kv head 0 codes 0..127, head 1 codes 128..255), so the output is the
    E4M3 value of every code (NaN for the two NaN codes), checked against the
    oracle's decoder."""
    Hq, Hkv, d = 8, 2, 128
    g = torch.Generator("cpu").manual_seed(5)
    q = torch.randn(1, Hq, d, generator=g).to(torch.bfloat16)
    k8 = torch.zeros(1, 4, Hkv, d, dtype=torch.uint8)
    k8[0, 0] = torch.randint(0, 0x70, (Hkv, d), generator=g, dtype=torch.uint8)
    v8 = torch.zeros(1, 4, Hkv, d, dtype=torch.uint8)
    v8[0, 0] = torch.arange(256, dtype=torch.int32).reshape(Hkv, d).to(torch.uint8)
    ones = torch.ones(Hkv)
    p = Params(64, 16, 1e4, 1.0 / math.sqrt(d), bifocal=bifocal)
    say("fp8 every code bifocal=%s" % bifocal)
    o, _ = jl.bifocal_decode_fp8(q.cuda(), k8.cuda(), v8.cuda(), ones, ones, [1], **_kw(p))
    torch.cuda.synchronize()
    want = np.array([oracle.e4m3_value(c) for c in range(256)]).reshape(Hkv, d)
    got = o.float().cpu().double().numpy()[0].reshape(Hkv, Hq // Hkv, d)
    for h in range(Hkv):
        for r in range(Hq // Hkv):
            assert np.array_equal(np.isnan(got[h, r]), np.isnan(want[h])), (h, r)
            ok = ~np.isnan(want[h])
            assert np.array_equal(got[h, r][ok], want[h][ok]), (h, r)


@pytest.mark.parametrize("B,S,Hq,Hkv,d,lens,w_pre,w_local", [
    (3, 1500, 8, 2, 128, [1500, 1, 777], 300, 100),   # mixed lengths, G = 5, 3, 1
    (1, 2600, 16, 2, 128, [2600], 700, 2200),          # GQA 8, window wider than a chunk
    (2, 900, 32, 2, 64, [900, 640], 256, 77),          # d = 64, GQA 16
])
def test_fp8_decode_vs_oracle(B, S, Hq, Hkv, d, lens, w_pre, w_local):
    q, k8, v8, ks, vs = inputs.decode_fp8_inputs(B, S, Hq, Hkv, d, seed=S + d)
    p = Params(w_pre, w_local, 1e4, 1.0 / math.sqrt(d))
    say("fp8 decode B=%d S=%d Hq=%d Hkv=%d d=%d lens=%s" % (B, S, Hq, Hkv, d, lens))
    k8d = k8.cuda()
    before = k8d.clone()
    o, lse = jl.bifocal_decode_fp8(q.cuda(), k8d, v8.cuda(), ks, vs, lens, **_kw(p))
    torch.cuda.synchronize()
    assert torch.equal(k8d, before), "the cache must never be rewritten"
    o_ref, lse_ref = oracle.decode_fp8(q, k8, v8, ks.numpy(), vs.numpy(), lens, **_kw(p))
    _check(o, lse, o_ref, lse_ref, "fp8 decode d=%d" % d)


@pytest.mark.parametrize("bifocal", [True, False])
def test_fp8_decode_128k(bifocal):
    q, k8, v8, ks, vs, lens, p = inputs.decode_fp8_128k()
    p = Params(p.w_pretrained, p.w_local, p.rope_base, p.softmax_scale, bifocal=bifocal)
    say("fp8 decode 128K bifocal=%s" % bifocal)
    o, lse = jl.bifocal_decode_fp8(q.cuda(), k8.cuda(), v8.cuda(), ks, vs, lens, **_kw(p))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_fp8(q, k8, v8, ks.numpy(), vs.numpy(), lens, **_kw(p))
    _check(o, lse, o_ref, lse_ref, "fp8 decode 128K bifocal=%s" % bifocal)


@pytest.mark.parametrize("page", [16, 128])
def test_fp8_paged_equals_flat(page):
    B, S, Hq, Hkv, d = 3, 1500, 8, 2, 128
    lens = [1500, 1, 777]
    q, k8, v8, ks, vs = inputs.decode_fp8_inputs(B, S, Hq, Hkv, d, seed=page)
    p = Params(300, 100, 1e4, 1.0 / math.sqrt(d))
    npp = [(L + page - 1) // page for L in lens]
    n_pages = sum(npp) + 2
    perm = np.random.default_rng(page).permutation(n_pages)
    kp = torch.zeros((n_pages, page, Hkv, d), dtype=torch.uint8)
    vp = torch.zeros_like(kp)
    bt = torch.full((B, max(npp) + 1), -5, dtype=torch.int32)
    nxt = 0
    for b, L in enumerate(lens):
        for pg in range(npp[b]):
            phys = int(perm[nxt])
            nxt += 1
            bt[b, pg] = phys
            r0, r1 = pg * page, min((pg + 1) * page, L)
            kp[phys, : r1 - r0] = k8[b, r0:r1]
            vp[phys, : r1 - r0] = v8[b, r0:r1]
    say("fp8 paged page=%d" % page)
    kw = dict(_kw(p), max_seqlen_k=max(lens))
    o_f, l_f = jl.bifocal_decode_fp8(q.cuda(), k8.cuda(), v8.cuda(), ks, vs, lens, **kw)
    o_p, l_p = jl.bifocal_decode_fp8(q.cuda(), kp.cuda(), vp.cuda(), ks, vs, lens,
                                     block_table=bt.cuda(), **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_f, o_p) and torch.equal(l_f, l_p)


def test_fp8_of_quantized_bf16_cache_tracks_bf16_decode():
    """End to end: a bf16 cache written to fp8 by jl_kv_quantize_fp8 and decoded
    gives the oracle's decode of the dequantized codes; its distance from the
    bf16 decode is the quantization error, not a kernel error."""
    q, kc, vc = inputs.decode_inputs(1, 3000, 8, 2, 128, seed=77)
    p = Params(1000, 300, 1e4, 1.0 / math.sqrt(128))
    ks = kc.float().abs().amax(dim=(0, 1, 3)) / 448.0
    vs = vc.float().abs().amax(dim=(0, 1, 3)) / 448.0
    k8 = jl.kv_quantize_fp8(kc.cuda(), ks.cuda())
    v8 = jl.kv_quantize_fp8(vc.cuda(), vs.cuda())
    o, lse = jl.bifocal_decode_fp8(q.cuda(), k8, v8, ks, vs, [3000], **_kw(p))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_fp8(q, k8.cpu(), v8.cpu(), ks.numpy(), vs.numpy(), [3000],
                                       **_kw(p))
    _check(o, lse, o_ref, lse_ref, "quantize + fp8 decode")

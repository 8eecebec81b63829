"""GPU parity of jl_bifocal_decode against the fp64 oracle, plus the decode
invariants: decode(p) == prefill row p, and the cache is never modified."""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_attention_jl_amd import inputs
from long_context_attention_jl_amd import jetlong as jl
from long_context_attention_jl_amd.inputs import Params

from _parity import TOL_BF16_LSE, TOL_BF16_O, TOL_F32_LSE, TOL_F32_O, say

pytestmark = pytest.mark.gpu


def _dec_gpu(q, kc, vc, lens, p, **kw):
    return jl.bifocal_decode(q.cuda(), kc, vc, lens, w_pretrained=p.w_pretrained,
                             w_local=p.w_local, rope_base=p.rope_base,
                             softmax_scale=p.softmax_scale, bifocal=p.bifocal, **kw)


def _dec_ref(q, kc, vc, lens, p):
    return oracle.decode(q, kc, vc, lens, w_pretrained=p.w_pretrained, w_local=p.w_local,
                         rope_base=p.rope_base, softmax_scale=p.softmax_scale, bifocal=p.bifocal)


def _check(o, lse, o_ref, lse_ref, dtype, label):
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    do, dl = np.abs(og - o_ref).max(), np.abs(lg - lse_ref).max()
    say("%s: max|dO|=%.3g max|dLSE|=%.3g" % (label, do, dl))
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    if dtype == torch.float32:
        assert do <= TOL_F32_O and dl <= TOL_F32_LSE, label
    else:
        assert do <= TOL_BF16_O and dl <= TOL_BF16_LSE, label


def test_decode_128k_workload():
    """32 q heads, 8 kv heads, d=128, cache of 131071 keys + the new token (L = 131072, G = 4)."""
    c = inputs.decode_128k()
    say("case", c.name)
    kc, vc = c.k_cache.cuda(), c.v_cache.cuda()
    k_before = kc.clone()
    o, lse = _dec_gpu(c.q, kc, vc, c.seqlens, c.params)
    torch.cuda.synchronize()
    assert torch.equal(kc, k_before), "the cache must never be rewritten"
    o_ref, lse_ref = _dec_ref(c.q, c.k_cache, c.v_cache, c.seqlens, c.params)
    _check(o, lse, o_ref, lse_ref, torch.bfloat16, c.name)
    # discrimination: bifocal differs from plain attention by far more than the error
    p0 = Params(c.params.w_pretrained, c.params.w_local, c.params.rope_base,
                c.params.softmax_scale, bifocal=False)
    o_pl, _ = _dec_ref(c.q, c.k_cache, c.v_cache, c.seqlens, p0)
    err = np.linalg.norm(o.float().cpu().double().numpy() - o_ref)
    assert np.linalg.norm(o_ref - o_pl) >= 10 * err


def test_decode_16_steps_across_g_switch():
    """Cache filled to 32760, then 16 steps append one token each: L = 32761..32776,
    G switches 1 -> 2 when L goes 32768 -> 32769; the cache is never rewritten."""
    queries, kc_h, vc_h, lens, p = inputs.decode_16step_cache()
    kc, vc = kc_h.cuda(), vc_h.cuda()
    snapshot = kc.clone()
    for step, (q, L) in enumerate(zip(queries, lens)):
        say("step", step, "L", L, "G", oracle.group_size(L, p.w_pretrained))
        o, lse = _dec_gpu(q, kc, vc, [L], p, max_seqlen_k=L)
        torch.cuda.synchronize()
        o_ref, lse_ref = _dec_ref(q, kc_h, vc_h, [L], p)
        _check(o, lse, o_ref, lse_ref, torch.bfloat16, "step %d L=%d" % (step, L))
    assert torch.equal(kc, snapshot)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
# (64, 12, 6): six waves, two of them with no SIMD partner in the tile-count
# balancing; (128, 24, 12): a second head group of four waves whose other
# four waves have no head
@pytest.mark.parametrize("d,Hq,Hkv", [(128, 8, 2), (64, 4, 4), (128, 16, 1), (64, 3, 1), (64, 12, 6),
                                      (128, 24, 12)])
def test_decode_small_batched(dtype, d, Hq, Hkv):
    B, S = 3, 700
    q, kc, vc = inputs.decode_inputs(B, S, Hq, Hkv, d, seed=d + Hq, dtype=dtype)
    lens = [700, 1, 333]
    p = Params(100, 50, 1e4, 1.0 / math.sqrt(d))
    say("small decode", dtype, d, Hq, Hkv)
    o, lse = _dec_gpu(q, kc.cuda(), vc.cuda(), lens, p)
    torch.cuda.synchronize()
    o_ref, lse_ref = _dec_ref(q, kc, vc, lens, p)
    _check(o, lse, o_ref, lse_ref, dtype, "small d=%d" % d)


@pytest.mark.parametrize("dtype,wgs", [(torch.float32, None), (torch.bfloat16, "2048")])
def test_decode_merge_of_many_chunks(dtype, wgs, monkeypatch):
    """More than 256 key chunks per sequence, so each merge thread folds
    several rounds of partials (fp32 caches aim at 512 workgroups; the bf16
    case raises the workgroup target through JL_DECODE_WGS)."""
    if wgs:
        monkeypatch.setenv("JL_DECODE_WGS", wgs)
    B, S, Hq, Hkv, d = 1, 40000, 8, 2, 128
    ws = jl.decode_workspace_bytes(B, S, Hq, Hkv, d, dtype)
    n_splits = ws // (B * Hq * (d + 2) * 4)
    say("many-chunk decode", dtype, "about", n_splits, "chunks")
    assert n_splits > 256
    q, kc, vc = inputs.decode_inputs(B, S, Hq, Hkv, d, seed=77, dtype=dtype)
    p = Params(8192, 2048, 1e6, 1.0 / math.sqrt(d))
    o, lse = _dec_gpu(q, kc.cuda(), vc.cuda(), [S], p)
    torch.cuda.synchronize()
    o_ref, lse_ref = _dec_ref(q, kc, vc, [S], p)
    _check(o, lse, o_ref, lse_ref, dtype, "many chunks %s" % dtype)


@pytest.mark.parametrize("label,p", [
    ("G1", Params(1000, 40, 1e4, 0.1)), ("w_local0", Params(64, 0, 1e4, 0.1)),
    ("w_local_all", Params(64, 4000, 1e4, 0.1)), ("plain", Params(64, 40, 1e4, 0.1, False)),
])
def test_decode_degenerate(label, p):
    q, kc, vc = inputs.decode_inputs(2, 900, 8, 2, 128, seed=31)
    lens = [900, 517]
    o, lse = _dec_gpu(q, kc.cuda(), vc.cuda(), lens, p)
    torch.cuda.synchronize()
    o_ref, lse_ref = _dec_ref(q, kc, vc, lens, p)
    _check(o, lse, o_ref, lse_ref, torch.bfloat16, label)


def test_decode_equals_prefill_last_row_on_gpu():
    """decode(p) over the cache prefill wrote (k_rot_out) equals prefill row p,
    across the G switch (w_pretrained = 600: G = 1 up to L = 600, then 2)."""
    T, Hq, Hkv, d = 1300, 4, 2, 128
    q, k, v = inputs.prefill_inputs(T, Hq, Hkv, d, seed=8)
    for L in (599, 600, 601, 1300):
        p = Params(600, 100, 1e6, 1.0 / math.sqrt(d))
        kr = torch.empty(L, Hkv, d, dtype=torch.bfloat16, device="cuda")
        o_p, l_p = jl.bifocal_prefill(q[:L].cuda(), k[:L].cuda(), v[:L].cuda(),
                                      w_pretrained=p.w_pretrained, w_local=p.w_local,
                                      rope_base=p.rope_base, softmax_scale=p.softmax_scale,
                                      k_rot_out=kr)
        o_d, l_d = _dec_gpu(q[L - 1:L], kr[None], v[:L].cuda()[None], [L], p)
        torch.cuda.synchronize()
        diff_o = (o_d[0].float() - o_p[L - 1].float()).abs().max().item()
        diff_l = (l_d[0] - l_p[:, L - 1]).abs().max().item()
        say("L=%d decode vs prefill: dO=%.3g dLSE=%.3g" % (L, diff_o, diff_l))
        assert diff_o <= TOL_BF16_O and diff_l <= TOL_BF16_LSE


def test_rope_apply_builds_the_cache_the_oracle_expects():
    """Cache rows written by jl_rope_apply (G = 1) decode like the oracle's
    fp64-rotated keys (within bf16 rounding of the stored rows)."""
    S, Hkv, d = 400, 2, 64
    _, k, v = inputs.prefill_inputs(S, 2, Hkv, d, seed=12)
    q = inputs.decode_query(1, 2, d, seed=13)
    kc = jl.rope_apply(k.cuda(), torch.arange(S), 1e4, G=1)
    p = Params(128, 30, 1e4, 0.125)
    o, lse = _dec_gpu(q, kc[None], v.cuda()[None], [S], p)
    torch.cuda.synchronize()
    o_ref, lse_ref = _dec_ref(q, kc[None].cpu(), v[None], [S], p)
    _check(o, lse, o_ref, lse_ref, torch.bfloat16, "rope_apply cache")

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

from _parity import TOL_BF16_LSE, TOL_BF16_O, TOL_F32_LSE, TOL_F32_O, check_decode, say

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


def _plain(p):
    return Params(p.w_pretrained, p.w_local, p.rope_base, p.softmax_scale, bifocal=False)


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
    # discrimination: bifocal differs from plain attention by far more than the error
    o_pl, _ = _dec_ref(c.q, c.k_cache, c.v_cache, c.seqlens, _plain(c.params))
    check_decode(o, lse, o_ref, lse_ref, torch.bfloat16, c.name, o_plain=o_pl)


def test_decode_128k_peaky():
    """The 128K decode with the query scaled by 4: a concentrated softmax, so
    the remote keys' fp16 correction rotation and the band edge show in o."""
    c = inputs.decode_128k()
    q = (c.q.float() * 4.0).to(torch.bfloat16)
    say("case", c.name, "q x4")
    o_ref, lse_ref = _dec_ref(q, c.k_cache, c.v_cache, c.seqlens, c.params)
    o_pl, _ = _dec_ref(q, c.k_cache, c.v_cache, c.seqlens, _plain(c.params))
    kc, vc = c.k_cache.cuda(), c.v_cache.cuda()
    for precise in (True, False):  # split-precision remote keys meet every bar
        o, lse = _dec_gpu(q, kc, vc, c.seqlens, c.params, precise=precise)
        torch.cuda.synchronize()
        check_decode(o, lse, o_ref, lse_ref, torch.bfloat16,
                     c.name + " q x4" + (" precise" if precise else ""), o_plain=o_pl,
                     check_lse=precise)


def test_decode_128k_sink_key():
    """The 128K decode with an attention sink: the query scores cache key 0
    about 13 above the other keys (through the lowest-frequency RoPE pairs),
    so one remote key carries about three quarters of the softmax.  Split precision meets
    every bar, the fast path the output bars (its LSE is recorded)."""
    c = inputs.decode_128k()
    q, kc = inputs.with_sink_key(c.q, c.k_cache, first_keys=[(0, 0)], q_add=3.0, k_value=6.1)
    q, kc = inputs.to_dtype(torch.bfloat16, q, kc)
    say("case", c.name, "sink key")
    o_ref, lse_ref = _dec_ref(q, kc, c.v_cache, c.seqlens, c.params)
    kcd, vcd = kc.cuda(), c.v_cache.cuda()
    for precise in (True, False):
        o, lse = _dec_gpu(q, kcd, vcd, c.seqlens, c.params, precise=precise)
        torch.cuda.synchronize()
        check_decode(o, lse, o_ref, lse_ref, torch.bfloat16,
                     c.name + " sink" + (" precise" if precise else ""), check_lse=precise)


@pytest.mark.parametrize("S", [131072, 3000])
def test_decode_large_magnitude_channels(S):
    """Cached keys with an outlier channel of magnitude 1e3..3e4 and values with
    outlier channels up to 6e4 (the fp16 operand range ends at 65504); the
    query is small in the channels the key outlier rotates into, so scores
    stay of order one.  The value channels' bar scales with their magnitude."""
    # the short cache takes a smaller pretraining window so that G > 1 there too
    p = inputs.DECODE_PARAMS if S > 65536 else Params(1024, 300, 1e6, 1.0 / math.sqrt(128))
    q, kc, vc = inputs.decode_inputs(1, S, 32, 8, 128, seed=404)
    q, kc, vc = inputs.with_outlier_channels(q, kc, vc, seed=405, q_small=7.0e-4)
    q, kc, vc = inputs.to_dtype(torch.bfloat16, q, kc, vc)
    scale = np.ones(128)
    vmax = vc.float().abs().amax(dim=(0, 1, 2)).double().numpy()
    for ch in inputs.outlier_value_channels(128):
        scale[ch] = vmax[ch]
    say("decode outliers S=%d max|k|=%.0f max|v|=%.0f" % (
        S, kc.float().abs().max().item(), vc.float().abs().max().item()))
    o_ref, lse_ref = _dec_ref(q, kc, vc, [S], p)
    o_pl, _ = _dec_ref(q, kc, vc, [S], _plain(p))
    kd, vd = kc.cuda(), vc.cuda()
    for precise in (True, False):
        o, lse = _dec_gpu(q, kd, vd, [S], p, precise=precise)
        torch.cuda.synchronize()
        check_decode(o, lse, o_ref, lse_ref, torch.bfloat16,
                     "decode outliers S=%d%s" % (S, " precise" if precise else ""),
                     o_plain=o_pl, o_scale=scale, check_lse=precise)


def test_decode_16_steps_across_g_switch():
    """Cache filled to 32760, then 16 steps append one token each: L = 32761..32776,
    G switches 1 -> 2 when L goes 32768 -> 32769; the cache is never rewritten."""
    queries, kc_h, vc_h, lens, p = inputs.decode_16step_cache()
    kc, vc = kc_h.cuda(), vc_h.cuda()
    snapshot = kc.clone()
    for step, (q, L) in enumerate(zip(queries, lens)):
        G = oracle.group_size(L, p.w_pretrained)
        say("step", step, "L", L, "G", G)
        o, lse = _dec_gpu(q, kc, vc, [L], p, max_seqlen_k=L)
        torch.cuda.synchronize()
        o_ref, lse_ref = _dec_ref(q, kc_h, vc_h, [L], p)
        o_pl = _dec_ref(q, kc_h, vc_h, [L], _plain(p))[0] if G > 1 else None
        check_decode(o, lse, o_ref, lse_ref, torch.bfloat16, "step %d L=%d" % (step, L),
                     o_plain=o_pl)
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


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_merge_of_many_chunks(dtype):
    """More than 256 key chunks per sequence (a 400000-key cache of two kv heads:
    bf16 chunks hold at most 32 stages of 48 positions, fp32 ones aim at 512
    workgroups), so the partials are folded over several rounds."""
    B, S, Hq, Hkv, d = 1, 400000, 8, 2, 128
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


@pytest.mark.parametrize("d,Hq,Hkv", [(128, 8, 2), (64, 16, 1), (128, 24, 12)])
def test_decode_precise_small_batched(d, Hq, Hkv):
    """Split-precision remote keys (precise = 1), flat and paged caches."""
    B, S = 3, 700
    q, kc, vc = inputs.decode_inputs(B, S, Hq, Hkv, d, seed=d + Hq + 5)
    lens = [700, 1, 333]
    p = Params(100, 50, 1e4, 1.0 / math.sqrt(d))
    say("precise decode", d, Hq, Hkv)
    o, lse = _dec_gpu(q, kc.cuda(), vc.cuda(), lens, p, precise=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = _dec_ref(q, kc, vc, lens, p)
    check_decode(o, lse, o_ref, lse_ref, torch.bfloat16, "precise d=%d" % d)
    # the same cache as pages of 64 rows in order
    page = 64
    npg = (S + page - 1) // page
    kp = torch.zeros(B * npg * page, Hkv, d, dtype=kc.dtype)
    vp = torch.zeros_like(kp)
    for b in range(B):
        kp[b * npg * page:b * npg * page + S] = kc[b]
        vp[b * npg * page:b * npg * page + S] = vc[b]
    bt = torch.arange(B * npg, dtype=torch.int32).view(B, npg)
    o2, l2 = jl.bifocal_decode_paged(q.cuda(), kp.view(-1, page, Hkv, d).cuda(),
                                     vp.view(-1, page, Hkv, d).cuda(), bt.cuda(), lens,
                                     w_pretrained=p.w_pretrained, w_local=p.w_local,
                                     rope_base=p.rope_base, softmax_scale=p.softmax_scale,
                                     precise=True, max_seqlen_k=S)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)


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


@pytest.mark.parametrize("L", [65535, 65536])
def test_decode_workgroup_target_boundary(L):
    """Flat bf16 caches of 65536 keys and more launch on the smaller workgroup
    target: 65535 keys take the default split and 65536 the smaller one.  Both
    against the oracle over every head, plus a batch of two where only the
    longer sequence reaches the boundary (max_seqlen_k decides the split)."""
    p = inputs.DECODE_PARAMS
    q, kc, vc = inputs.decode_inputs(2, L, 32, 8, 128, seed=L)
    lens = [L, L // 3]
    o, lse = _dec_gpu(q, kc.cuda(), vc.cuda(), lens, p, max_seqlen_k=L)
    o_ref, lse_ref = _dec_ref(q, kc, vc, lens, p)
    o_pl, _ = _dec_ref(q, kc, vc, lens, _plain(p))
    check_decode(o, lse, o_ref, lse_ref, torch.bfloat16, "decode boundary L=%d" % L, o_plain=o_pl)

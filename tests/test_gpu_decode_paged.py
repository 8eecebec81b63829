"""GPU parity of jl_bifocal_decode_paged: the cache pool is the flat cache's
rows scattered over shuffled pages, so the paged decode must give the flat
decode's results (same arithmetic, other addresses) and match the fp64
oracle.  Where both assign the keys to workgroups alike (short caches: one
stage per workgroup) they agree bit for bit; on long flat caches the
workgroups take interleaved stages, so the partial sums group differently
and the two agree to rounding."""
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


def _paginate(kc, vc, lens, page, seed):
    """Flat caches [B, S, Hkv, d] -> shuffled page pools and a block table.
    Table slots past a sequence's pages hold out-of-range numbers: they must
    never be read."""
    B, S, Hkv, d = kc.shape
    npp = [(L + page - 1) // page for L in lens]
    stride = max(npp) + 2
    n_pages = sum(npp) + 3  # a few spare pages the table never names
    perm = np.random.default_rng(seed).permutation(n_pages)
    kp = torch.zeros((n_pages, page, Hkv, d), dtype=kc.dtype)
    vp = torch.zeros_like(kp)
    bt = torch.full((B, stride), -7, dtype=torch.int32)
    bt[:, -1] = 1 << 30
    nxt = 0
    for b, L in enumerate(lens):
        for pg in range(npp[b]):
            phys = int(perm[nxt])
            nxt += 1
            bt[b, pg] = phys
            r0, r1 = pg * page, min((pg + 1) * page, L)
            kp[phys, : r1 - r0] = kc[b, r0:r1]
            vp[phys, : r1 - r0] = vc[b, r0:r1]
    return kp, vp, bt


def _run_both(q, kc, vc, lens, p, page, seed):
    kp, vp, bt = _paginate(kc, vc, lens, page, seed)
    kw = dict(w_pretrained=p.w_pretrained, w_local=p.w_local, rope_base=p.rope_base,
              softmax_scale=p.softmax_scale, bifocal=p.bifocal, max_seqlen_k=max(lens))
    o_f, l_f = jl.bifocal_decode(q.cuda(), kc.cuda(), vc.cuda(), lens, **kw)
    o_p, l_p = jl.bifocal_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), bt.cuda(), lens, **kw)
    torch.cuda.synchronize()
    return o_f, l_f, o_p, l_p


def _close_to_flat(o_f, l_f, o_p, l_p, label):
    """Paged against flat with another grouping of the partial sums: the
    outputs may differ by the rounding of their last bits only."""
    do = (o_f.float() - o_p.float()).abs().max().item()
    dl = (l_f - l_p).abs().max().item()
    say("%s: paged vs flat max|dO|=%.3g max|dLSE|=%.3g" % (label, do, dl))
    assert do <= 2.0 ** -7 * max(o_f.float().abs().max().item(), 1e-3), label  # one bf16 ulp
    assert dl <= 1e-5 * max(l_f.abs().max().item(), 1.0), label


def _oracle(q, kc, vc, lens, p):
    return oracle.decode(q, kc, vc, lens, w_pretrained=p.w_pretrained, w_local=p.w_local,
                         rope_base=p.rope_base, softmax_scale=p.softmax_scale, bifocal=p.bifocal)


@pytest.mark.parametrize("page,Hq,Hkv,d", [(16, 8, 2, 128), (64, 8, 2, 128), (256, 8, 2, 128),
                                          (32, 32, 2, 64)])
def test_paged_equals_flat_and_oracle(page, Hq, Hkv, d):
    B, S = 3, 1500
    lens = [1500, 1, 777]
    q, kc, vc = inputs.decode_inputs(B, S, Hq, Hkv, d, seed=page)
    p = Params(300, 100, 1e4, 1.0 / math.sqrt(d))
    say("paged decode page=%d Hq=%d Hkv=%d d=%d lens=%s" % (page, Hq, Hkv, d, lens))
    o_f, l_f, o_p, l_p = _run_both(q, kc, vc, lens, p, page, seed=page)
    assert torch.equal(o_f, o_p) and torch.equal(l_f, l_p), "paged differs from flat"
    o_ref, l_ref = _oracle(q, kc, vc, lens, p)
    do = np.abs(o_p.float().cpu().double().numpy() - o_ref).max()
    dl = np.abs(l_p.cpu().double().numpy() - l_ref).max()
    say("paged page=%d: max|dO|=%.3g max|dLSE|=%.3g" % (page, do, dl))
    assert do <= TOL_BF16_O and dl <= TOL_BF16_LSE


def test_paged_128k_and_g_switch():
    """The 128K decode workload (G = 4) and the G 1 -> 2 crossing on pages of 64 rows."""
    c = inputs.decode_128k()
    p = c.params
    say("paged decode", c.name)
    o_f, l_f, o_p, l_p = _run_both(c.q, c.k_cache, c.v_cache, c.seqlens, p, 64, seed=1)
    _close_to_flat(o_f, l_f, o_p, l_p, "paged 128K")
    o_ref, l_ref = _oracle(c.q, c.k_cache, c.v_cache, c.seqlens, p)
    dl = np.abs(l_p.cpu().double().numpy() - l_ref).max()
    say("paged 128K: max|dLSE|=%.3g" % dl)
    assert dl <= TOL_BF16_LSE
    queries, kc, vc, lens, p = inputs.decode_16step_cache()
    for step in (7, 8):  # L = 32768 (G = 1) and 32769 (G = 2)
        o_f, l_f, o_p, l_p = _run_both(queries[step], kc, vc, [lens[step]], p, 64, seed=step)
        _close_to_flat(o_f, l_f, o_p, l_p, "step %d" % step)

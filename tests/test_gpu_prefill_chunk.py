"""GPU parity of jl_bifocal_prefill_chunk (and its paged form) against the fp64
oracle: a chunk of new rows per sequence attends to every key of its
sequence in a cache of standard-RoPE keys, with G from the sequence's
length.  Small cases compare every row (unaligned chunk starts, rows on both
sides of the split-precision boundary 2048, packed batches with an empty
chunk, a G switch inside the batch); the 128K chunk runs at full size and
compares a row sample."""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_attention_jl_amd import inputs
from long_context_attention_jl_amd import jetlong as jl
from long_context_attention_jl_amd.inputs import Params

from _parity import check_prefill, say

pytestmark = pytest.mark.gpu


def _kw(p, bifocal=None):
    return dict(w_pretrained=p.w_pretrained, w_local=p.w_local, rope_base=p.rope_base,
                softmax_scale=p.softmax_scale, bifocal=p.bifocal if bifocal is None else bifocal)


def _gpu(q, kc, vc, lens, cu, p, **extra):
    o, lse = jl.bifocal_prefill_chunk(q.cuda(), kc.cuda(), vc.cuda(), lens, cu_seqlens_q=cu,
                                      **_kw(p), **extra)
    torch.cuda.synchronize()
    return o, lse


def _oracle(q, kc, vc, lens, cu, p, rows=None):
    return oracle.prefill_chunk(q, kc, vc, lens, cu_seqlens_q=cu, rows=rows, **_kw(p))


def _paginate(kc, vc, lens, page, seed):
    """Flat caches [B, S, Hkv, d] -> page pools in shuffled order and a block
    table; entries past a sequence's pages hold out-of-range numbers."""
    B, S, Hkv, d = kc.shape
    npp = [(L + page - 1) // page for L in lens]
    stride = max(npp) + 1
    n_pages = sum(npp) + 2
    perm = np.random.default_rng(seed).permutation(n_pages)
    kp = torch.zeros((n_pages, page, Hkv, d), dtype=kc.dtype)
    vp = torch.zeros_like(kp)
    bt = torch.full((B, stride), 1 << 30, dtype=torch.int32)
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


@pytest.mark.parametrize("L,C,Hq,Hkv,d,w_pre,w_local", [
    (1500, 700, 8, 2, 128, 300, 100),    # unaligned chunk start, G = 5
    (1500, 1500, 4, 2, 128, 300, 100),   # the whole sequence as one chunk
    (1500, 1, 4, 2, 128, 300, 100),      # one row (the decode case)
    (3000, 1000, 4, 1, 128, 1024, 300),  # rows on both sides of 2048, GQA 4
    (2600, 555, 2, 2, 64, 700, 2200),    # d = 64, window wider than a workgroup
    (300, 300, 2, 2, 64, 100, 40),       # split-precision rows only, d = 64
])
def test_chunk_full_rows(L, C, Hq, Hkv, d, w_pre, w_local):
    p = Params(w_pre, w_local, 1e4, 1.0 / math.sqrt(d))
    q, kc, vc, _ = inputs.chunk_inputs([C], [L], L + 5, Hq, Hkv, d, seed=L + C + d)
    say("chunk L=%d C=%d Hq=%d Hkv=%d d=%d %s" % (L, C, Hq, Hkv, d, p))
    kc_before = kc.clone()
    o, lse = _gpu(q, kc, vc, [L], None, p)
    o_ref, lse_ref = _oracle(q, kc, vc, [L], None, p)
    check_prefill(o, lse, o_ref, lse_ref, list(range(C)), torch.bfloat16, "chunk L=%d C=%d" % (L, C))
    assert torch.equal(kc, kc_before)


def test_chunk_batch_with_empty_chunk_and_g_switch():
    """Three sequences: 2600 keys with 900 new rows (G = 3), 1100 keys with none,
    and 1024 keys with all 1024 new (G = 1, bifocal inactive) -- w_pretrained 1024."""
    lens, chunks = [2600, 1100, 1024], [900, 0, 1024]
    p = Params(1024, 256, 1e4, 1.0 / math.sqrt(128))
    q, kc, vc, cu = inputs.chunk_inputs(chunks, lens, 2700, 8, 2, 128, seed=41)
    say("chunk batch lens=%s chunks=%s" % (lens, chunks))
    o, lse = _gpu(q, kc, vc, lens, cu, p)
    o_ref, lse_ref = _oracle(q, kc, vc, lens, cu, p)
    check_prefill(o, lse, o_ref, lse_ref, list(range(sum(chunks))), torch.bfloat16, "chunk batch")


@pytest.mark.parametrize("page", [16, 64, 256])
def test_chunk_paged_equals_flat(page):
    lens, chunks = [2600, 1100, 777], [900, 0, 777]
    p = Params(1024, 256, 1e4, 1.0 / math.sqrt(128))
    q, kc, vc, cu = inputs.chunk_inputs(chunks, lens, 2700, 8, 2, 128, seed=43)
    say("chunk paged page=%d" % page)
    o_f, l_f = _gpu(q, kc, vc, lens, cu, p)
    kp, vp, bt = _paginate(kc, vc, lens, page, seed=page)
    o_p, l_p = jl.bifocal_prefill_chunk_paged(q.cuda(), kp.cuda(), vp.cuda(), bt.cuda(), lens,
                                              cu_seqlens_q=cu, **_kw(p))
    torch.cuda.synchronize()
    assert torch.equal(o_f, o_p) and torch.equal(l_f, l_p), "paged differs from flat"
    o_ref, lse_ref = _oracle(q, kc, vc, lens, cu, p)
    check_prefill(o_p, l_p, o_ref, lse_ref, list(range(sum(chunks))), torch.bfloat16,
                  "chunk paged %d" % page)


@pytest.mark.parametrize("mode", ["not_bifocal", "w_local_0", "w_local_wide"])
def test_chunk_degenerate_settings(mode):
    L, C = 1800, 600
    w_local = {"not_bifocal": 200, "w_local_0": 0, "w_local_wide": 5000}[mode]
    p = Params(400, w_local, 1e4, 1.0 / math.sqrt(128), bifocal=mode != "not_bifocal")
    q, kc, vc, _ = inputs.chunk_inputs([C], [L], L, 4, 2, 128, seed=47)
    say("chunk degenerate", mode)
    o, lse = _gpu(q, kc, vc, [L], None, p)
    o_ref, lse_ref = _oracle(q, kc, vc, [L], None, p)
    check_prefill(o, lse, o_ref, lse_ref, list(range(C)), torch.bfloat16, "chunk " + mode)


def test_chunk_128k_sampled():
    """4096 new rows on a 131072-key sequence (G = 4) in the benchmark's launch
    configuration; a row sample against the oracle, and the last row against
    the decode entry point (the same query at the same position)."""
    c = inputs.chunk_128k()
    say("case", c.name)
    o, lse = _gpu(c.q, c.k_cache, c.v_cache, c.seqlens, None, c.params)
    C = c.q.shape[0]
    rows = sorted({0, 1, 2, 63, 64, 255, 256, 1000, 2047, 2048, 2049, 3000, C - 2, C - 1})
    o_ref, lse_ref = _oracle(c.q, c.k_cache, c.v_cache, c.seqlens, None, c.params, rows=rows)
    check_prefill(o, lse, o_ref, lse_ref, rows, torch.bfloat16, c.name)
    o_d, l_d = jl.bifocal_decode(c.q[C - 1:].cuda(), c.k_cache.cuda(), c.v_cache.cuda(),
                                 c.seqlens, **_kw(c.params))
    torch.cuda.synchronize()
    assert (o_d[0].float() - o[C - 1].float()).abs().max().item() <= 2e-2
    assert abs(l_d[0] - lse[:, C - 1]).max().item() <= 1e-3


def test_chunk_invalid_device_lengths_write_nothing():
    """seqlens_k below the chunk size breaks the contract: the plan zeroes every
    length, so the outputs keep their sentinel."""
    q, kc, vc, cu = inputs.chunk_inputs([300, 200], [700, 500], 800, 2, 1, 64, seed=3)
    p = Params(300, 64, 1e4, 0.125)
    o = torch.full_like(q, 7.0).cuda()
    lse = torch.full((2, 500), 7.0, device="cuda")
    jl.bifocal_prefill_chunk(q.cuda(), kc.cuda(), vc.cuda(), [700, 150], cu_seqlens_q=cu,
                             max_seqlen_q=300, max_seqlen_k=700, out=o, lse_out=lse, **_kw(p))
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())


def test_chunk_1024_rows_key_split_128k():
    """1024 new rows on a 131072-key sequence: 128 row-block workgroups, so each
    row block's keys are split in four shares merged in LogSumExp space."""
    q, kc, vc, _ = inputs.chunk_inputs([1024], [131072], 131072, 32, 8, 128, seed=66)
    p = inputs.DECODE_PARAMS
    say("chunk 1024 rows on 131072 keys (key split)")
    o, lse = _gpu(q, kc, vc, [131072], None, p)
    rows = [0, 1, 255, 256, 511, 700, 1022, 1023]
    o_ref, lse_ref = _oracle(q, kc, vc, [131072], None, p, rows=rows)
    check_prefill(o, lse, o_ref, lse_ref, rows, torch.bfloat16, "chunk1024 split")


def test_chunk_precise_full_rows_and_key_split_off():
    """Split precision (precise = 1) on a chunk whose rows cross 2048 and on a
    1024-row chunk of a long cache (which would otherwise split its keys in
    shares): every row against the oracle."""
    for L, C, Hq, Hkv, d, w_pre, w_local in ((3100, 1500, 4, 2, 128, 1000, 300),
                                              (9000, 1024, 32, 8, 128, 2048, 700)):
        p = Params(w_pre, w_local, 1e4, 1.0 / math.sqrt(d))
        q, kc, vc, _ = inputs.chunk_inputs([C], [L], L, Hq, Hkv, d, seed=L + C + 3)
        say("precise chunk L=%d C=%d" % (L, C))
        o, lse = _gpu(q, kc, vc, [L], None, p, precise=True)
        o_ref, lse_ref = _oracle(q, kc, vc, [L], None, p)
        check_prefill(o, lse, o_ref, lse_ref, list(range(C)), torch.bfloat16,
                      "precise chunk L=%d C=%d" % (L, C))


def _ws(Tq, B, max_k, Hq, Hkv, d, precise=False):
    return torch.empty(jl.prefill_chunk_workspace_bytes(Tq, B, max_k, Hq, Hkv, d, precise),
                       dtype=torch.uint8, device="cuda")


def _chunk_step(q, kc, vc, lens, chunks, p, ws, reuse, max_k, **extra):
    cu = [0]
    for c in chunks:
        cu.append(cu[-1] + c)
    o, lse = jl.bifocal_prefill_chunk(q, kc, vc, lens, cu_seqlens_q=cu, max_seqlen_k=max_k,
                                      workspace=ws, reuse_images=reuse, **_kw(p), **extra)
    torch.cuda.synchronize()
    return o.clone(), lse.clone(), cu


def test_chunk_reuse_images_across_a_chunked_prefill():
    """Two sequences grow over five chunk calls on one kept workspace with
    reuse_images: G changes between calls (1 -> 2 -> 3 for the first, w_pretrained
    1024), the second sequence skips a call (no new rows: its images must
    survive) and then resumes.  Every call equals a call that rebuilds all
    images on a fresh workspace, bit for bit; the last also meets the oracle."""
    Hq, Hkv, d, S, max_k = 8, 2, 128, 2700, 2700
    p = Params(1024, 256, 1e4, 1.0 / math.sqrt(d))
    steps = [([700, 1100], [700, 1100]), ([1400, 1500], [700, 400]), ([2100, 1500], [700, 0]),
             ([2400, 1800], [300, 300]), ([2600, 1900], [200, 100])]
    _, kc, vc, _ = inputs.chunk_inputs([1], [S, S], S, Hq, Hkv, d, seed=71)
    g = torch.Generator("cpu").manual_seed(72)
    kcd, vcd = kc.cuda(), vc.cuda()
    ws = _ws(max(sum(c) for _, c in steps), 2, max_k, Hq, Hkv, d)
    for i, (lens, chunks) in enumerate(steps):
        q = (torch.randn(sum(chunks), Hq, d, generator=g)).to(torch.bfloat16)
        say("reuse step %d lens=%s chunks=%s" % (i, lens, chunks))
        # the first call of a prefill rebuilds: the workspace may hold images
        # of other caches that happened to sit at the same addresses
        o_r, l_r, cu = _chunk_step(q.cuda(), kcd, vcd, lens, chunks, p, ws, i > 0, max_k)
        o_f, l_f, _ = _chunk_step(q.cuda(), kcd, vcd, lens, chunks, p,
                                  _ws(sum(chunks), 2, max_k, Hq, Hkv, d), False, max_k)
        assert torch.equal(o_r, o_f) and torch.equal(l_r, l_f), "step %d" % i
    o_ref, lse_ref = _oracle(q, kc, vc, lens, cu, p)
    check_prefill(o_r, l_r, o_ref, lse_ref, list(range(sum(chunks))), torch.bfloat16,
                  "chunk reuse last step")


@pytest.mark.parametrize("case", ["other_cache", "rewritten_rows_no_reuse", "interp", "paged",
                                  "precise"])
def test_chunk_reuse_images_invalidation(case):
    """Images are rebuilt whenever they may not hold: another cache (same
    shapes) under reuse_images, rows rewritten in place with reuse_images off,
    continuous interpolation (bifocal 2) at a new length; and kept on paged
    caches and with split precision.  Each call equals a fresh rebuild."""
    Hq, Hkv, d, L0, L1, max_k = 4, 2, 128, 1300, 1900, 2000
    p = Params(600, 200, 1e4, 1.0 / math.sqrt(d), bifocal=2 if case == "interp" else 1)
    extra = dict(precise=True) if case == "precise" else {}
    _, kc, vc, _ = inputs.chunk_inputs([1], [max_k], max_k, Hq, Hkv, d, seed=73)
    g = torch.Generator("cpu").manual_seed(74)
    q0 = torch.randn(L0 - 100, Hq, d, generator=g).to(torch.bfloat16).cuda()
    q1 = torch.randn(L1 - L0, Hq, d, generator=g).to(torch.bfloat16).cuda()
    kcd, vcd = kc.cuda(), vc.cuda()
    pre = case == "precise"
    ws = _ws(L0, 1, max_k, Hq, Hkv, d, pre)
    say("reuse invalidation", case)

    if case == "paged":  # one pool for every call (the images name it by address)
        pools = [t.cuda() for t in _paginate(kc, vc, [max_k], 64, seed=5)]

    def run(kk, vv, q, L, wsx, reuse):
        if case == "paged":
            kp, vp, bt = pools
            o, lse = jl.bifocal_prefill_chunk_paged(q, kp, vp, bt, [L], max_seqlen_k=max_k,
                                                    workspace=wsx, reuse_images=reuse,
                                                    **_kw(p), **extra)
        else:
            o, lse = jl.bifocal_prefill_chunk(q, kk, vv, [L], max_seqlen_k=max_k, workspace=wsx,
                                              reuse_images=reuse, **_kw(p), **extra)
        torch.cuda.synchronize()
        return o.clone(), lse.clone()

    run(kcd, vcd, q0, L0, ws, False)
    if case == "other_cache":
        kcd, vcd = (kcd * 0.5).contiguous(), (vcd + 1.0).contiguous()
        reuse = True
    elif case == "rewritten_rows_no_reuse":
        kcd[:, :500] *= -1.0
        reuse = False
    else:
        reuse = True
    o_r, l_r = run(kcd, vcd, q1, L1, ws, reuse)
    o_f, l_f = run(kcd, vcd, q1, L1, _ws(L1 - L0, 1, max_k, Hq, Hkv, d, pre), False)
    assert torch.equal(o_r, o_f) and torch.equal(l_r, l_f), case
    if case in ("other_cache", "rewritten_rows_no_reuse", "interp"):
        o_ref, lse_ref = _oracle(q1.cpu(), kcd.cpu(), vcd.cpu(), [L1], None, p)
        check_prefill(o_r, l_r, o_ref, lse_ref, list(range(L1 - L0)), torch.bfloat16,
                      "reuse " + case)


def test_chunk_reuse_images_1024_rows_128k():
    """The benchmark's chunked step: 1024 rows at L = 131072 after a call that
    built the images of the first 130048 keys (same G = 4) on the kept
    workspace; equals a rebuild bit for bit."""
    q, kc, vc, _ = inputs.chunk_inputs([2048], [131072], 131072, 32, 8, 128, seed=67)
    p = inputs.DECODE_PARAMS
    L = 131072
    qd, kcd, vcd = q.cuda(), kc.cuda(), vc.cuda()
    ws = _ws(1024, 1, L, 32, 8, 128)
    say("chunk reuse 1024 rows on 131072 keys")
    _chunk_step(qd[:1024].contiguous(), kcd, vcd, [L - 1024], [1024], p, ws, False, L)
    o_r, l_r, _ = _chunk_step(qd[1024:].contiguous(), kcd, vcd, [L], [1024], p, ws, True, L)
    o_f, l_f, _ = _chunk_step(qd[1024:].contiguous(), kcd, vcd, [L], [1024], p,
                              _ws(1024, 1, L, 32, 8, 128), False, L)
    assert torch.equal(o_r, o_f) and torch.equal(l_r, l_f)

"""A seeded sweep of random settings against the fp64 oracle: packed sequences
of random lengths, head counts and group sizes, both head sizes, random
pretrained and local windows, the three RoPE modes (plain, bifocal,
continuous interpolation), split precision, and for decode flat, paged and
fp8 caches.  Every row (prefill) and every head (decode) is compared; the
cases are drawn once from a fixed generator, so every run sees the same list."""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_attention_jl_amd import inputs
from long_context_attention_jl_amd import jetlong as jl

from _parity import check_decode, check_prefill, say

pytestmark = pytest.mark.gpu


def _prefill_cases(n=40, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        n_seqs = int(rng.integers(1, 4))
        lens = [int(x) for x in rng.integers(1, 1400, size=n_seqs)]
        if i % 4 == 0:
            lens[0] = int(rng.integers(2049, 3200))  # rows >= 2048 reach the main kernel
        Hkv = int(rng.choice([1, 2, 4]))
        Hq = Hkv * int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        w_pre = int(rng.integers(8, 2500))
        w_local = int(rng.integers(0, 2600))
        mode = int(rng.choice([0, 1, 1, 2]))
        precise = bool(mode != 0 and rng.random() < 0.25)
        dtype = torch.float32 if (i % 7 == 3) else torch.bfloat16
        if dtype == torch.float32:  # the fp32 path has no split precision or interpolation
            precise = False
            mode = min(mode, 1)
        out.append((i, lens, Hq, Hkv, d, w_pre, w_local, mode, precise, dtype))
    return out


@pytest.mark.parametrize("case", _prefill_cases(), ids=lambda c: "p%d" % c[0])
def test_prefill_sweep(case):
    i, lens, Hq, Hkv, d, w_pre, w_local, mode, precise, dtype = case
    T = sum(lens)
    cu = [0] + list(np.cumsum(lens))
    q, k, v = inputs.prefill_inputs(T, Hq, Hkv, d, seed=100 + i, dtype=dtype, q_scale=1.0 / math.sqrt(d))
    kw = dict(w_pretrained=w_pre, w_local=w_local, rope_base=1e4, softmax_scale=1.0,
              bifocal=mode)
    say("sweep prefill %d: lens=%s Hq=%d Hkv=%d d=%d w_pre=%d w_local=%d mode=%d precise=%s %s"
        % (i, lens, Hq, Hkv, d, w_pre, w_local, mode, precise, dtype))
    o, lse = jl.bifocal_prefill(q.cuda(), k.cuda(), v.cuda(), cu_seqlens=cu,
                                **(dict(kw, precise=True) if precise else kw))
    torch.cuda.synchronize()
    rows = list(range(T))
    o_ref, l_ref = oracle.prefill(q, k, v, cu_seqlens=cu, rows=rows, **kw)
    check_prefill(o, lse, o_ref, l_ref, rows, dtype, "sweep prefill %d" % i)


def _decode_cases(n=32, seed=7):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 5))
        lens = [int(x) for x in rng.integers(1, 6000, size=B)]
        if i % 5 == 0:
            lens[-1] = int(rng.integers(20000, 40000))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        Hq = Hkv * int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        w_pre = int(rng.integers(8, 6000))
        w_local = int(rng.integers(0, 3000))
        mode = int(rng.choice([0, 1, 1, 2]))
        cache = str(rng.choice(["flat", "paged", "fp8"]))
        precise = bool(mode != 0 and cache != "fp8" and rng.random() < 0.3)
        out.append((i, lens, Hq, Hkv, d, w_pre, w_local, mode, cache, precise))
    return out


@pytest.mark.parametrize("case", _decode_cases(), ids=lambda c: "d%d" % c[0])
def test_decode_sweep(case):
    i, lens, Hq, Hkv, d, w_pre, w_local, mode, cache, precise = case
    B, S = len(lens), max(lens)
    kw = dict(w_pretrained=w_pre, w_local=w_local, rope_base=1e4, softmax_scale=1.0 / math.sqrt(d),
              bifocal=mode)
    say("sweep decode %d: lens=%s Hq=%d Hkv=%d d=%d w_pre=%d w_local=%d mode=%d %s precise=%s"
        % (i, lens, Hq, Hkv, d, w_pre, w_local, mode, cache, precise))
    if cache == "fp8":
        q, k8, v8, ks, vs = inputs.decode_fp8_inputs(B, S, Hq, Hkv, d, seed=200 + i)
        o, lse = jl.bifocal_decode_fp8(q.cuda(), k8.cuda(), v8.cuda(), ks.cuda(), vs.cuda(), lens, **kw)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.decode_fp8(q, k8, v8, ks.numpy(), vs.numpy(), lens, **kw)
        check_decode(o, lse, o_ref, l_ref, torch.bfloat16, "sweep decode %d" % i)
        return
    q, kc, vc = inputs.decode_inputs(B, S, Hq, Hkv, d, seed=200 + i)
    if cache == "flat":
        o, lse = jl.bifocal_decode(q.cuda(), kc.cuda(), vc.cuda(), lens, precise=precise, **kw)
    else:
        page = 16 if i % 2 else 64
        npg = (S + page - 1) // page
        perm = torch.randperm(B * npg, generator=torch.Generator().manual_seed(i))
        kp = torch.zeros(B * npg, page, Hkv, d, dtype=kc.dtype)
        vp = torch.zeros_like(kp)
        bt = torch.empty(B, npg, dtype=torch.int32)
        for b in range(B):
            for j in range(npg):
                dst = int(perm[b * npg + j])
                bt[b, j] = dst
                rows = kc[b, j * page:min((j + 1) * page, S)]
                kp[dst, :rows.shape[0]] = rows
                vp[dst, :rows.shape[0]] = vc[b, j * page:min((j + 1) * page, S)]
        o, lse = jl.bifocal_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), bt.cuda(), lens,
                                         precise=precise, max_seqlen_k=S, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode(q, kc, vc, lens, **kw)
    check_decode(o, lse, o_ref, l_ref, torch.bfloat16, "sweep decode %d" % i)


def _chunk_cases(n=32, seed=99):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 4))
        lens = [int(x) for x in rng.integers(1, 4000, size=B)]
        chunks = [int(rng.integers(0, L + 1)) if rng.random() < 0.8 else 0 for L in lens]
        if sum(chunks) == 0:
            chunks[0] = lens[0]
        Hkv = int(rng.choice([1, 2, 4]))
        Hq = Hkv * int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        w_pre = int(rng.integers(8, 3000))
        w_local = int(rng.integers(0, 2500))
        mode = int(rng.choice([0, 1, 1, 2]))
        precise = bool(mode != 0 and rng.random() < 0.25)
        paged = bool(rng.random() < 0.4)
        reuse = bool(not precise and rng.random() < 0.5)
        out.append((i, lens, chunks, Hq, Hkv, d, w_pre, w_local, mode, precise, paged, reuse))
    return out


def _pages(kc, vc, lens, page, seed):
    B, S, Hkv, d = kc.shape
    npp = [max((L + page - 1) // page, 1) for L in lens]
    stride = max(npp)
    n_pages = sum(npp)
    perm = np.random.default_rng(seed).permutation(n_pages)
    kp = torch.zeros((n_pages, page, Hkv, d), dtype=kc.dtype)
    vp = torch.zeros_like(kp)
    bt = torch.zeros((B, stride), dtype=torch.int32)
    nxt = 0
    for b, L in enumerate(lens):
        for pg in range(npp[b]):
            phys = int(perm[nxt])
            nxt += 1
            bt[b, pg] = phys
            r0, r1 = pg * page, min((pg + 1) * page, L)
            if r1 > r0:
                kp[phys, : r1 - r0] = kc[b, r0:r1]
                vp[phys, : r1 - r0] = vc[b, r0:r1]
    return kp, vp, bt


@pytest.mark.parametrize("case", _chunk_cases(), ids=lambda c: "c%d" % c[0])
def test_chunk_sweep(case):
    """Chunks of random sizes (some empty) appended to caches of random
    lengths; with reuse, an earlier call on the same workspace saw the caches
    before the chunk (its own G), and the call under test keeps its images."""
    i, lens, chunks, Hq, Hkv, d, w_pre, w_local, mode, precise, paged, reuse = case
    S = max(lens) + 3
    q, kc, vc, cu = inputs.chunk_inputs(chunks, lens, S, Hq, Hkv, d, seed=300 + i)
    cu = [int(x) for x in cu]
    kw = dict(w_pretrained=w_pre, w_local=w_local, rope_base=1e4, softmax_scale=1.0 / math.sqrt(d),
              bifocal=mode)
    say("sweep chunk %d: lens=%s chunks=%s Hq=%d Hkv=%d d=%d w_pre=%d w_local=%d mode=%d "
        "precise=%s paged=%s reuse=%s" % (i, lens, chunks, Hq, Hkv, d, w_pre, w_local, mode,
                                          precise, paged, reuse))
    extra = dict(precise=precise, max_seqlen_k=max(lens))
    ws = torch.empty(jl.prefill_chunk_workspace_bytes(max(sum(chunks), 1), len(lens), max(lens), Hq, Hkv, d,
                                                      precise=precise),
                     dtype=torch.uint8, device="cuda")
    if paged:
        page = 16 if i % 2 else 64
        kp, vp, bt = _pages(kc, vc, lens, page, seed=i)
        kpd, vpd, btd = kp.cuda(), vp.cuda(), bt.cuda()

        def call(ll, qq, cc, **more):
            return jl.bifocal_prefill_chunk_paged(qq.cuda(), kpd, vpd, btd, ll, cu_seqlens_q=cc,
                                                  workspace=ws, **kw, **extra, **more)
    else:
        kcd, vcd = kc.cuda(), vc.cuda()

        def call(ll, qq, cc, **more):
            return jl.bifocal_prefill_chunk(qq.cuda(), kcd, vcd, ll, cu_seqlens_q=cc, workspace=ws,
                                            **kw, **extra, **more)
    kept = False
    if reuse:
        # the previous step: each sequence without its new rows (at least one key)
        prev = [max(L - c, 1) for L, c in zip(lens, chunks)]
        pch = [min(c, pl) for c, pl in zip(chunks, prev)]
        if sum(pch) > 0:
            pcu = [0] + [int(x) for x in np.cumsum(pch)]
            call(prev, q[:sum(pch)], pcu, reuse_images=False)
            torch.cuda.synchronize()
            kept = True
    o, lse = call(lens, q, cu, reuse_images=kept)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.prefill_chunk(q, kc, vc, lens, cu_seqlens_q=cu, **kw)
    check_prefill(o, lse, o_ref, l_ref, list(range(sum(chunks))), torch.bfloat16, "sweep chunk %d" % i)


def _three_cases(n=12, seed=5):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        lens = [int(x) for x in rng.integers(1, 2600, size=int(rng.integers(1, 3)))]
        Hkv = int(rng.choice([1, 2, 4]))
        Hq = Hkv * int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        w_pre = int(rng.integers(8, 2000))
        w_local = int(rng.integers(0, 2600))
        out.append((i, lens, Hq, Hkv, d, w_pre, w_local))
    return out


@pytest.mark.parametrize("case", _three_cases(), ids=lambda c: "t%d" % c[0])
def test_three_call_sweep(case):
    """The pages' unfused form (three calls and the LogSumExp merge), prefill
    and decode, against the oracle's direct definition."""
    i, lens, Hq, Hkv, d, w_pre, w_local = case
    T = sum(lens)
    cu = [0] + [int(x) for x in np.cumsum(lens)]
    kw = dict(w_pretrained=w_pre, w_local=w_local, rope_base=1e4, softmax_scale=1.0)
    say("sweep three-call %d: lens=%s Hq=%d Hkv=%d d=%d w_pre=%d w_local=%d"
        % (i, lens, Hq, Hkv, d, w_pre, w_local))
    q, k, v = inputs.prefill_inputs(T, Hq, Hkv, d, seed=400 + i, q_scale=1.0 / math.sqrt(d))
    o, lse = jl.bifocal_prefill_three_call(q.cuda(), k.cuda(), v.cuda(), cu_seqlens=cu, **kw)
    torch.cuda.synchronize()
    rows = list(range(T))
    o_ref, l_ref = oracle.prefill(q, k, v, cu_seqlens=cu, rows=rows, **kw)
    check_prefill(o, lse, o_ref, l_ref, rows, torch.bfloat16, "sweep three-call prefill %d" % i)
    # decode: one query per sequence against caches of the same lengths
    B, S = len(lens), max(lens)
    qd, kc, vc = inputs.decode_inputs(B, S, Hq, Hkv, d, seed=500 + i)
    kwd = dict(kw, softmax_scale=1.0 / math.sqrt(d))
    od, ld = jl.bifocal_decode_three_call(qd.cuda(), kc.cuda(), vc.cuda(), lens, **kwd)
    torch.cuda.synchronize()
    od_ref, ld_ref = oracle.decode(qd, kc, vc, lens, **kwd)
    check_decode(od, ld, od_ref, ld_ref, torch.bfloat16, "sweep three-call decode %d" % i)

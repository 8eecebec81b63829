"""GPU parity of jl_bifocal_prefill against the fp64 oracle.

Small cases compare every row (several tiles, ragged tails, both the
split-precision rows < 2048 and the main kernel's rows >= 2048); the named
long-context workloads run at full size in the benchmark's launch
configuration and compare a deterministic row sample the oracle computes
one row at a time."""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_attention_jl_amd import inputs
from long_context_attention_jl_amd import jetlong as jl
from long_context_attention_jl_amd.inputs import Params

from _parity import (block_rows, check_prefill, gpu_prefill, oracle_prefill_rows,
                     sample_rows, say)

pytestmark = pytest.mark.gpu


def _full_case(T, Hq, Hkv, d, params, dtype=torch.bfloat16, seed=0, cu=None, q_scale=None):
    q, k, v = inputs.prefill_inputs(T, Hq, Hkv, d, seed=seed, dtype=dtype,
                                    q_scale=1.0 if q_scale is None else q_scale)
    say("case T=%d Hq=%d Hkv=%d d=%d %s cu=%s params=%s" % (T, Hq, Hkv, d, dtype, cu, params))
    o, lse = gpu_prefill(jl, q, k, v, params, cu=cu)
    torch.cuda.synchronize()
    rows = list(range(T))
    o_ref, lse_ref = oracle_prefill_rows(q, k, v, params, rows, cu=cu)
    return check_prefill(o, lse, o_ref, lse_ref, rows, dtype, "T=%d d=%d" % (T, d))


def test_tiny_f32_workload_full():
    """1 head, d=64, L=512, w_pretrained=128 (G=4), w_local=32, fp32: every row."""
    c = inputs.tiny_prefill()
    say("case", c.name)
    o, lse = gpu_prefill(jl, c.q, c.k, c.v, c.params)
    rows = list(range(c.T))
    o_ref, lse_ref = oracle_prefill_rows(c.q, c.k, c.v, c.params, rows)
    o_pl, _ = oracle_prefill_rows(c.q, c.k, c.v, c.params, rows, bifocal=False)
    check_prefill(o, lse, o_ref, lse_ref, rows, torch.float32, c.name, o_plain=o_pl)


@pytest.mark.parametrize("T,Hq,Hkv,d,w_pre,w_local", [
    (700, 4, 2, 128, 200, 96),     # G=4, ragged tail, straddling tiles
    (333, 2, 2, 64, 100, 40),      # d=64
    (3000, 4, 1, 128, 1024, 300),  # rows >= 2048 reach the main kernel, GQA 4
    (2600, 2, 2, 64, 700, 2200),   # main kernel, d=64, window wider than a workgroup
])
def test_bf16_small_full(T, Hq, Hkv, d, w_pre, w_local):
    p = Params(w_pre, w_local, 1e4, 1.0 / math.sqrt(d))
    _full_case(T, Hq, Hkv, d, p, seed=T + d)


@pytest.mark.parametrize("T,Hq,Hkv,d,w_pre,w_local,cu", [
    (3000, 4, 1, 128, 1024, 300, None),              # rows >= 2048 in split precision too
    (2600, 2, 2, 64, 700, 2200, None),
    (3563, 4, 2, 128, 256, 90, [0, 300, 301, 1000, 3500, 3563]),
])
def test_bf16_precise_full(T, Hq, Hkv, d, w_pre, w_local, cu):
    """Split precision on every row (precise = 1): every row against the oracle."""
    p = Params(w_pre, w_local, 1e4, 1.0 / math.sqrt(d))
    q, k, v = inputs.prefill_inputs(T, Hq, Hkv, d, seed=T + d + 1)
    say("precise T=%d d=%d cu=%s" % (T, d, cu))
    o, lse = gpu_prefill(jl, q, k, v, p, cu=cu, precise=True)
    torch.cuda.synchronize()
    rows = list(range(T))
    o_ref, lse_ref = oracle_prefill_rows(q, k, v, p, rows, cu=cu)
    check_prefill(o, lse, o_ref, lse_ref, rows, torch.bfloat16, "precise T=%d" % T)


@pytest.mark.parametrize("T,d", [(700, 128), (2300, 64)])
def test_f32_small_full(T, d):
    p = Params(256, 77, 1e4, 1.0 / math.sqrt(d))
    _full_case(T, 2, 1, d, p, dtype=torch.float32, seed=7)


def test_f32_varlen_edges_and_settings():
    """The fp32 kernel across its row blocks and phases: packed sequences of
    lengths 300, 1, 699, 2500 and 63 (G = 2, 1, 3, 10, 1), then the degenerate
    windows (every key remote, every key local, plain RoPE), every row."""
    cu = [0, 300, 301, 1000, 3500, 3563]
    _full_case(cu[-1], 4, 2, 128, Params(256, 90, 1e4, 1.0 / math.sqrt(128)), dtype=torch.float32,
               seed=9, cu=cu)
    for p in (Params(300, 0, 1e4, 0.125), Params(300, 5000, 1e4, 0.125),
              Params(300, 64, 1e4, 0.125, bifocal=False)):
        _full_case(1100, 2, 1, 64, p, dtype=torch.float32, seed=10)


@pytest.mark.parametrize("label,params", [
    ("G1", Params(4096, 64, 1e4, 0.125)),          # L <= w_pretrained: plain RoPE
    ("w_local0", Params(300, 0, 1e4, 0.125)),      # every key remote (call B alone)
    ("w_local_all", Params(300, 5000, 1e4, 0.125)),  # every key local
    ("not_bifocal", Params(300, 64, 1e4, 0.125, bifocal=False)),
    ("w_local1", Params(250, 1, 1e4, 0.125)),      # only the diagonal is local
])
def test_bf16_degenerate_settings(label, params):
    say("degenerate", label)
    _full_case(2200, 2, 1, 64, params, seed=11)


def test_bf16_varlen_small():
    cu = [0, 300, 301, 1000, 3500, 3563]
    p = Params(256, 90, 1e4, 1.0 / math.sqrt(128))
    _full_case(cu[-1], 4, 2, 128, p, seed=5, cu=cu)


def test_single_token_and_edge_lengths():
    for T in (1, 2, 63, 64, 65, 255, 256, 257):
        _full_case(T, 2, 1, 128, Params(16, 3, 1e4, 0.1), seed=T)


def test_g1_equals_plain_on_gpu():
    """[BT] §3.1: with G = 1 the bifocal result is plain RoPE attention (same kernels)."""
    q, k, v = inputs.prefill_inputs(3000, 2, 1, 128, seed=3)
    p1 = Params(4096, 100, 1e6, 0.088)
    p0 = Params(4096, 100, 1e6, 0.088, bifocal=False)
    o1, l1 = gpu_prefill(jl, q, k, v, p1)
    o0, l0 = gpu_prefill(jl, q, k, v, p0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o0) and torch.equal(l1, l0)


def test_boundary_probe_closed_form_gpu():
    """The pages' band edge through the GPU: q = e_0, one key kappa*e_0 at
    distance w_local (remote) or w_local - 1 (local), all other keys 0.  The
    LSE then equals ln(i + exp(s * kappa * cos(distance))) with the distance
    measured in standard or remapped positions -- a closed form, not the oracle."""
    L, w_pre, w_local, d = 64, 16, 7, 64
    G = 4
    scale, kappa = 1.0, 2.0
    checked = 0
    for i in range(w_local, L):
        for jstar, remote in ((i - w_local, True), (i - w_local + 1, False)):
            d_std, d_rem = i - jstar, i // G - jstar // G
            want = math.log(i + math.exp(kappa * math.cos(d_rem if remote else d_std)))
            other = math.log(i + math.exp(kappa * math.cos(d_std if remote else d_rem)))
            if abs(want - other) < 0.05:
                continue
            q = torch.zeros(L, 1, d, dtype=torch.bfloat16)
            q[:, 0, 0] = 1.0
            k = torch.zeros(L, 1, d, dtype=torch.bfloat16)
            k[jstar, 0, 0] = kappa
            v = torch.zeros(L, 1, d, dtype=torch.bfloat16)
            _, lse = gpu_prefill(jl, q, k, v, Params(w_pre, w_local, 1e4, scale))
            got = float(lse[0, i].item())
            assert abs(got - want) < 1e-3, (i, jstar, got, want, other)
            checked += 1
    assert checked >= 20


def test_poisoned_outputs_are_fully_written_and_deterministic():
    q, k, v = inputs.prefill_inputs(2600, 4, 2, 128, seed=9)
    p = Params(700, 200, 1e4, 0.088)
    outs = []
    for _ in range(3):
        o = torch.full((2600, 4, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((4, 2600), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.full((jl.prefill_workspace_bytes(2600, 1, 4, 2, 128, torch.bfloat16),),
                        255, dtype=torch.uint8, device="cuda")
        gpu_prefill(jl, q, k, v, p, out=o, lse_out=lse, workspace=ws)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        outs.append((o.clone(), lse.clone()))
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


def test_k_rot_out_is_standard_rope():
    q, k, v = inputs.prefill_inputs(500, 2, 2, 128, seed=4)
    kr = torch.empty(500, 2, 128, dtype=torch.bfloat16, device="cuda")
    gpu_prefill(jl, q, k, v, Params(100, 20, 1e6, 0.1), k_rot_out=kr)
    torch.cuda.synchronize()
    ref = oracle.rope(k, np.arange(500), 1e6)
    got = kr.float().cpu().double().numpy()
    assert np.abs(got - ref).max() <= 2.0 ** -8 * np.abs(ref).max()


# ---- the named long-context workloads at full size --------------------------
# One row of every 256-row block of every sequence (every prefill workgroup,
# since all heads are compared), plus the band-edge, split-precision and
# group-boundary rows; the oracle computes them one by one.

def _rows_of(case, every=1, n_strided=12):
    """(rows, mask of rows whose sequence has G > 1)."""
    rows, big = [], []
    cu = case.cu_seqlens or [0, case.T]
    for a, b in zip(cu[:-1], cu[1:]):
        L = b - a
        G = oracle.group_size(L, case.params.w_pretrained)
        r = set(block_rows(L, a)[::every])
        r.update(a + x for x in sample_rows(L, case.params.w_local, G, n_strided=n_strided))
        r = sorted(r)
        rows += r
        big += [G > 1] * len(r)
    return rows, np.array(big, dtype=bool)


def _plain_on(case, rows, mask, o_ref):
    """The oracle's plain-RoPE output on the rows of `mask` (o_ref elsewhere)."""
    o_plain = o_ref.copy()
    sel = [r for r, m in zip(rows, mask) if m]
    if sel:
        o_pl, _ = oracle_prefill_rows(case.q, case.k, case.v, case.params, sel,
                                      cu=case.cu_seqlens, bifocal=False)
        o_plain[mask] = o_pl
    return o_plain


def _full_size(case, label, every=1, o_scale=None, modes=(False,), disc=True):
    """modes: the precise flags to run; the fast path (False) on concentrated
    attention has its LSE recorded, not asserted (see check_prefill).
    disc=False skips the discrimination ratio (inputs on which bifocal and
    plain attention nearly agree)."""
    rows, mask = _rows_of(case, every)
    say("workload", case.name, label, "- comparing %d rows x %d heads" % (len(rows), case.q.shape[1]))
    o_ref, lse_ref = oracle_prefill_rows(case.q, case.k, case.v, case.params, rows,
                                         cu=case.cu_seqlens)
    o_plain = _plain_on(case, rows, mask, o_ref) if disc else None
    out = None
    for precise in modes:
        o, lse = gpu_prefill(jl, case.q, case.k, case.v, case.params, cu=case.cu_seqlens,
                             precise=precise)
        torch.cuda.synchronize()
        strict = precise or len(modes) == 1
        check_prefill(o, lse, o_ref, lse_ref, rows, case.q.dtype,
                      label + (" precise" if precise else ""), o_plain=o_plain, disc_rows=mask,
                      o_scale=o_scale, check_lse=strict)
        out = (o, lse) if out is None else out
        del o, lse
    return out


def test_qwen3_1p7b_65536_every_workgroup():
    _full_size(inputs.qwen3_1p7b_64k(), "qwen3_1p7b_L65536")


def test_qwen3_8b_131072_every_workgroup():
    _full_size(inputs.qwen3_8b_128k(), "qwen3_8b_L131072")


def test_qwen3_8b_131072_peaky():
    """The 128K layer with q scaled by 4 (scores of standard deviation 4: the
    softmax concentrates on a few keys, so the fp16 probabilities and the
    band edge show at the output level).  One row of every 512-row block."""
    c = inputs.qwen3_8b_128k()
    c.q = (c.q.float() * 4.0).to(torch.bfloat16)
    _full_size(c, "qwen3_8b_L131072 q x4", every=2, modes=(True, False))


def test_varlen_4seq_every_workgroup_and_g1_sequences_plain():
    c = inputs.varlen_4seq()
    o, lse = _full_size(c, "varlen_4seq")
    # sequences with G = 1 equal plain RoPE causal attention
    p0 = Params(c.params.w_pretrained, c.params.w_local, c.params.rope_base,
                c.params.softmax_scale, bifocal=False)
    o0, l0 = gpu_prefill(jl, c.q, c.k, c.v, p0, cu=c.cu_seqlens)
    torch.cuda.synchronize()
    for s in range(2):  # lengths 8192 and 32768 (G = 1)
        a, b = c.cu_seqlens[s], c.cu_seqlens[s + 1]
        assert torch.equal(o[a:b], o0[a:b]) and torch.equal(lse[:, a:b], l0[:, a:b])
    # and the G > 1 sequences differ from plain attention
    a, b = c.cu_seqlens[3], c.cu_seqlens[4]
    assert (lse[:, a:b] - l0[:, a:b]).abs().max().item() > 1e-3


def test_sink_key_full():
    """An attention sink: every query scores key 0 about 9 above the other keys
    (through the lowest-frequency RoPE pairs, so at every position), so key 0
    carries about three quarters of a long row's softmax -- a remote key for
    the rows past the local window.  Every row; split precision meets every bar, the fast
    path the output bars (its LSE is recorded).  Bifocal and plain attention
    nearly agree here (both are dominated by the same key), so there is no
    discrimination ratio."""
    p = Params(1024, 300, 1e4, 1.0)
    q, k, v = inputs.prefill_inputs(3000, 4, 2, 128, seed=61, q_scale=1.0 / math.sqrt(128))
    q, k = inputs.with_sink_key(q, k, first_keys=[0], q_add=0.4, k_value=2.8)
    q, k, v = inputs.to_dtype(torch.bfloat16, q, k, v)
    say("sink key T=3000")
    rows = list(range(3000))
    o_ref, lse_ref = oracle_prefill_rows(q, k, v, p, rows)
    for precise in (True, False):
        o, lse = gpu_prefill(jl, q, k, v, p, precise=precise)
        torch.cuda.synchronize()
        check_prefill(o, lse, o_ref, lse_ref, rows, torch.bfloat16,
                      "sink T=3000" + (" precise" if precise else ""), check_lse=precise)


def test_sink_key_128k():
    """The 128K layer with an attention sink at key 0 (as test_sink_key_full,
    scored about 13 above the rest, about three quarters of the mass of the
    last rows): one row of every 1024-row block plus the band-edge rows, both
    precisions."""
    base = inputs.qwen3_8b_128k()
    q, k = inputs.with_sink_key(base.q, base.k, first_keys=[0], q_add=0.5, k_value=3.25)
    q, k = inputs.to_dtype(torch.bfloat16, q, k)
    case = inputs.PrefillCase(base.name + "_sink", q, k, base.v, None, base.params)
    del base
    _full_size(case, "qwen3_8b_L131072 sink", every=4, modes=(True, False), disc=False)


def _outlier_case(T, Hq, Hkv, d, seed, params, q_scale, q_small):
    q, k, v = inputs.prefill_inputs(T, Hq, Hkv, d, seed=seed, q_scale=q_scale)
    q, k, v = inputs.with_outlier_channels(q, k, v, seed=seed + 1, q_small=q_small)
    q, k, v = inputs.to_dtype(torch.bfloat16, q, k, v)
    scale = np.ones(d)
    vmax = v.float().abs().amax(dim=(0, 1)).double().numpy()
    for c in inputs.outlier_value_channels(d):
        scale[c] = vmax[c]
    return q, k, v, scale


@pytest.mark.parametrize("T,Hq,Hkv,d,w_pre,w_local", [
    (3000, 4, 2, 128, 1024, 300),  # both kernels (rows below and above 2048), ragged tail
    (1300, 2, 1, 64, 400, 100),
])
def test_large_magnitude_channels_full(T, Hq, Hkv, d, w_pre, w_local):
    """Keys with an outlier channel up to 3e4 and values with outlier channels
    up to 6e4 (near the fp16 operand limit of 65504), every row compared.
    The value channels' bar scales with their magnitude (attention is linear
    in v channel by channel).  Split precision meets every bar; the fast path
    meets the output bars (its LSE error is recorded)."""
    p = Params(w_pre, w_local, 1e4, 1.0)
    q, k, v, scale = _outlier_case(T, Hq, Hkv, d, 40 + d, p, 1.0 / math.sqrt(d), 7.0e-5)
    say("outliers T=%d d=%d max|k|=%.0f max|v|=%.0f" % (
        T, d, k.float().abs().max().item(), v.float().abs().max().item()))
    rows = list(range(T))
    o_ref, lse_ref = oracle_prefill_rows(q, k, v, p, rows)
    o_pl, _ = oracle_prefill_rows(q, k, v, p, rows, bifocal=False)
    for precise in (True, False):
        o, lse = gpu_prefill(jl, q, k, v, p, precise=precise)
        torch.cuda.synchronize()
        check_prefill(o, lse, o_ref, lse_ref, rows, torch.bfloat16,
                      "outliers T=%d%s" % (T, " precise" if precise else ""), o_plain=o_pl,
                      o_scale=scale, check_lse=precise)


def test_large_magnitude_channels_128k():
    """The 128K layer's shape with outlier key and value channels: one row of
    every 1024-row block plus the band-edge rows."""
    base = inputs.qwen3_8b_128k()
    q, k, v = inputs.with_outlier_channels(base.q, base.k, base.v, seed=303, q_small=7.0e-5)
    q, k, v = inputs.to_dtype(torch.bfloat16, q, k, v)
    case = inputs.PrefillCase(base.name + "_outliers", q, k, v, None, base.params)
    del base
    scale = np.ones(q.shape[2])
    vmax = v.float().abs().amax(dim=(0, 1)).double().numpy()
    for c in inputs.outlier_value_channels(q.shape[2]):
        scale[c] = vmax[c]
    _full_size(case, "qwen3_8b_L131072 outlier channels", every=4, o_scale=scale,
               modes=(True, False))


def test_operands_beyond_fp16_range_are_not_clamped():
    """The bf16 path's MFMA operands are fp16: a rotated key beyond 65504 is
    not clamped to a finite value.  A row that scores it comes out
    non-finite, so the failure shows; rows that never see that key are
    unaffected and match the oracle."""
    T, d, jbad = 300, 64, 200
    p = Params(128, 32, 1e4, 1.0)
    q, k, v = inputs.prefill_inputs(T, 1, 1, d, seed=99, q_scale=1.0 / math.sqrt(d))
    q[jbad, 0, :] = 0.0
    q[jbad, 0, 0] = 1.0  # the row at jbad scores its own key with standard RoPE: q . k
    k[jbad, 0, :] = 0.0
    k[jbad, 0, 0] = 1.0e5  # bf16 99840: beyond fp16 once rotated into either channel
    o, lse = gpu_prefill(jl, q, k, v, p)
    torch.cuda.synchronize()
    row_ok = torch.isfinite(o.float()).all(dim=(1, 2)) & torch.isfinite(lse).all(dim=0)
    assert not bool(row_ok[jbad]), "a row scoring an out-of-range key must not look finite"
    rows = list(range(jbad))
    o_ref, lse_ref = oracle_prefill_rows(q, k, v, p, rows)
    check_prefill(o, lse, o_ref, lse_ref, rows, torch.bfloat16, "rows before the bad key")

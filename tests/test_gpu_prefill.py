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

from _parity import (check_prefill, gpu_prefill, oracle_prefill_rows, sample_rows,
                     say)

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
    check_prefill(o, lse, o_ref, lse_ref, rows, torch.float32, c.name)


@pytest.mark.parametrize("T,Hq,Hkv,d,w_pre,w_local", [
    (700, 4, 2, 128, 200, 96),     # G=4, ragged tail, straddling tiles
    (333, 2, 2, 64, 100, 40),      # d=64
    (3000, 4, 1, 128, 1024, 300),  # rows >= 2048 reach the main kernel, GQA 4
    (2600, 2, 2, 64, 700, 2200),   # main kernel, d=64, window wider than a workgroup
])
def test_bf16_small_full(T, Hq, Hkv, d, w_pre, w_local):
    p = Params(w_pre, w_local, 1e4, 1.0 / math.sqrt(d))
    _full_case(T, Hq, Hkv, d, p, seed=T + d)


@pytest.mark.parametrize("T,d", [(700, 128), (2300, 64)])
def test_f32_small_full(T, d):
    p = Params(256, 77, 1e4, 1.0 / math.sqrt(d))
    _full_case(T, 2, 1, d, p, dtype=torch.float32, seed=7)


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


# ---- the named long-context workloads at full size (sampled rows) -------------

def _sampled(case, label, discrimination=False):
    say("workload", case.name)
    o, lse = gpu_prefill(jl, case.q, case.k, case.v, case.params, cu=case.cu_seqlens)
    torch.cuda.synchronize()
    rows = []
    cu = case.cu_seqlens or [0, case.T]
    for a, b in zip(cu[:-1], cu[1:]):
        G = oracle.group_size(b - a, case.params.w_pretrained)
        rows += [a + r for r in sample_rows(b - a, case.params.w_local, G, n_strided=12)]
    o_ref, lse_ref = oracle_prefill_rows(case.q, case.k, case.v, case.params, rows,
                                         cu=case.cu_seqlens)
    o_plain = None
    if discrimination:
        o_plain, _ = oracle_prefill_rows(case.q, case.k, case.v, case.params, rows,
                                         cu=case.cu_seqlens, bifocal=False)
    check_prefill(o, lse, o_ref, lse_ref, rows, case.q.dtype, label, o_plain=o_plain)
    return o, lse


def test_qwen3_1p7b_65536_sampled():
    _sampled(inputs.qwen3_1p7b_64k(), "qwen3_1p7b_L65536")


def test_qwen3_8b_131072_sampled():
    _sampled(inputs.qwen3_8b_128k(), "qwen3_8b_L131072", discrimination=True)


def test_varlen_4seq_sampled_and_g1_sequences_plain():
    c = inputs.varlen_4seq()
    o, lse = _sampled(c, "varlen_4seq")
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

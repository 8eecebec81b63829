"""Shared helpers of the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle

# Parity bars: fp32 inputs max |dO| <= 1e-4; bf16 inputs (fp32 accumulation)
# max |dO| <= 2e-2 and max |dLSE| <= 1e-3.  G, f and band membership bit-exact.
TOL_F32_O = 1e-4
TOL_F32_LSE = 1e-4
TOL_BF16_O = 2e-2
TOL_BF16_LSE = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def sample_rows(L: int, w_local: int, G: int, n_strided: int = 32, seed: int = 0):
    """Deterministic row sample of one sequence: the first rows, both sides of
    the band edge, the split-precision boundary (2048), group boundaries, the
    last rows and evenly strided rows."""
    s = set(range(0, min(L, 24)))
    for c in (w_local, 2048, 4096, L // 2, L - 1):
        for dlt in range(-3, 4):
            if 0 <= c + dlt < L:
                s.add(c + dlt)
    for k in (1, 7, 1000, 10007):
        x = k * G
        for dlt in (-1, 0, 1):
            if 0 <= x + dlt < L:
                s.add(x + dlt)
    s.update(range(max(0, L - 8), L))
    s.update(int(x) for x in np.linspace(0, L - 1, n_strided))
    rng = np.random.default_rng(seed)
    s.update(int(x) for x in rng.integers(0, L, size=8))
    return sorted(s)


def check_prefill(o_gpu, lse_gpu, o_ref, lse_ref, rows, dtype, label, o_plain=None):
    """o_gpu [T, Hq, d] / lse_gpu [Hq, T] (device); o_ref [R, Hq, d] / lse_ref
    [R, Hq] (oracle, fp64) for the global rows `rows`."""
    idx = torch.as_tensor(rows, dtype=torch.long, device=o_gpu.device)
    og = o_gpu.index_select(0, idx).float().cpu().double().numpy()
    lg = lse_gpu.index_select(1, idx).cpu().double().numpy().T
    do = np.abs(og - o_ref)
    dl = np.abs(lg - lse_ref)
    assert np.isfinite(og).all() and np.isfinite(lg).all(), label + ": non-finite output"
    rel = float(np.linalg.norm(og - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
    msg = "%s: max|dO|=%.3g max|dLSE|=%.3g relRMS=%.3g rows=%d" % (
        label, do.max(), dl.max(), rel, len(rows))
    if o_plain is not None:
        disc = float(np.linalg.norm(o_ref - o_plain) / max(np.linalg.norm(og - o_ref), 1e-300))
        msg += " discrimination=%.1f" % disc
    say(msg)
    if dtype == torch.float32:
        assert do.max() <= TOL_F32_O, msg
        assert dl.max() <= TOL_F32_LSE, msg
    else:
        assert do.max() <= TOL_BF16_O, msg
        assert dl.max() <= TOL_BF16_LSE, msg
    if o_plain is not None:
        assert disc >= 10.0, msg
    return do.max(), dl.max()


def oracle_prefill_rows(case_q, case_k, case_v, params, rows, cu=None, bifocal=None, threads=0):
    kw = dict(w_pretrained=params.w_pretrained, w_local=params.w_local,
              rope_base=params.rope_base, softmax_scale=params.softmax_scale,
              bifocal=params.bifocal if bifocal is None else bifocal)
    return oracle.prefill(case_q, case_k, case_v, cu_seqlens=cu, rows=rows, n_threads=threads, **kw)


def gpu_prefill(jl, q, k, v, params, cu=None, **extra):
    return jl.bifocal_prefill(q.cuda(), k.cuda(), v.cuda(), w_pretrained=params.w_pretrained,
                              w_local=params.w_local, rope_base=params.rope_base,
                              softmax_scale=params.softmax_scale, bifocal=params.bifocal,
                              cu_seqlens=cu, **extra)


def ln_sum_exp(xs):
    m = max(xs)
    return m + math.log(sum(math.exp(x - m) for x in xs))

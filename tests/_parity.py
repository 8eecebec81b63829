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
# Relative RMS error ||O_gpu - O_ref|| / ||O_ref||.  Storing O in bf16 (round
# to nearest even, relative error at most 2^-9 of the value's binade) alone
# gives about 2^-9 / sqrt(3) = 1.1e-3; the fp16 MFMA operands add errors of
# the same order.  The bar is 3.5 times the storage rounding.  fp32 inputs run
# in fp32 throughout: rounding there is near 2^-24 per operation.
REL_RMS_BF16 = 4e-3
REL_RMS_F32 = 1e-5
# ||O_bifocal - O_plain|| / ||O_gpu - O_bifocal|| on rows whose sequence has
# G > 1: the comparison must see the difference the method makes.
DISC_MIN = 10.0


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


def block_rows(L: int, start: int = 0):
    """One row of every 256-row block of a sequence of L positions (the rows of
    one prefill workgroup), offset by `start` tokens.  The 32-row slot (the
    wave) and the row within it move from block to block, so across a long
    sequence every wave slot and every lane position is compared."""
    rows = []
    for b in range((L + 255) // 256):
        r = 256 * b + 32 * (b % 8) + (13 * b) % 32
        rows.append(start + min(r, L - 1))
    return rows


def check_prefill(o_gpu, lse_gpu, o_ref, lse_ref, rows, dtype, label, o_plain=None,
                  disc_rows=None, o_scale=None, check_lse=True):
    """o_gpu [T, Hq, d] / lse_gpu [Hq, T] (device); o_ref [R, Hq, d] / lse_ref
    [R, Hq] (oracle, fp64) for the global rows `rows`.

    o_plain: the oracle's plain-RoPE output on the same rows; the
    discrimination ratio is then asserted over the rows where `disc_rows`
    (a boolean mask over `rows`, default all) is true.
    o_scale: per-channel scale [d] of the values.  Attention is linear in v,
    channel by channel, so the output bar for values of scale s_c is the
    unit-scale bar times s_c.
    check_lse=False records the LSE error without asserting it (the fast
    fp16-operand path on concentrated attention; the split-precision path
    is held to the bar)."""
    idx = torch.as_tensor(rows, dtype=torch.long, device=o_gpu.device)
    og = o_gpu.index_select(0, idx).float().cpu().double().numpy()
    lg = lse_gpu.index_select(1, idx).cpu().double().numpy().T
    do = np.abs(og - o_ref)
    if o_scale is not None:
        do = do / np.asarray(o_scale, dtype=np.float64).reshape(1, 1, -1)
    dl = np.abs(lg - lse_ref)
    assert np.isfinite(og).all() and np.isfinite(lg).all(), label + ": non-finite output"
    rel = float(np.linalg.norm(og - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
    msg = "%s: max|dO|=%.3g max|dLSE|=%.3g relRMS=%.3g rows=%d" % (
        label, do.max(), dl.max(), rel, len(rows))
    disc = None
    if o_plain is not None:
        m = np.ones(len(rows), dtype=bool) if disc_rows is None else np.asarray(disc_rows, bool)
        disc = float(np.linalg.norm(o_ref[m] - o_plain[m]) /
                     max(np.linalg.norm(og[m] - o_ref[m]), 1e-300))
        msg += " discrimination=%.1f" % disc
    say(msg)
    if dtype == torch.float32:
        assert do.max() <= TOL_F32_O, msg
        assert dl.max() <= TOL_F32_LSE, msg
        assert rel <= REL_RMS_F32, msg
    else:
        assert do.max() <= TOL_BF16_O, msg
        assert dl.max() <= TOL_BF16_LSE or not check_lse, msg
        assert rel <= REL_RMS_BF16, msg
    if disc is not None:
        assert disc >= DISC_MIN, msg
    return do.max(), dl.max()


def check_decode(o, lse, o_ref, lse_ref, dtype, label, o_plain=None, o_scale=None,
                 check_lse=True):
    """Decode outputs o [B, Hq, d] / lse [B, Hq] (device) against the oracle's
    (fp64): the same bars as check_prefill, over every head of every sequence."""
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    do = np.abs(og - o_ref)
    if o_scale is not None:
        do = do / np.asarray(o_scale, dtype=np.float64).reshape(1, 1, -1)
    dl = np.abs(lg - lse_ref)
    assert np.isfinite(og).all() and np.isfinite(lg).all(), label + ": non-finite output"
    rel = float(np.linalg.norm(og - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
    msg = "%s: max|dO|=%.3g max|dLSE|=%.3g relRMS=%.3g" % (label, do.max(), dl.max(), rel)
    disc = None
    if o_plain is not None:
        disc = float(np.linalg.norm(o_ref - o_plain) / max(np.linalg.norm(og - o_ref), 1e-300))
        msg += " discrimination=%.1f" % disc
    say(msg)
    if dtype == torch.float32:
        assert do.max() <= TOL_F32_O and dl.max() <= TOL_F32_LSE and rel <= REL_RMS_F32, msg
    else:
        assert do.max() <= TOL_BF16_O and rel <= REL_RMS_BF16, msg
        assert dl.max() <= TOL_BF16_LSE or not check_lse, msg
    if disc is not None:
        assert disc >= DISC_MIN, msg
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

"""Pins for the fp64 CPU oracle: checks against what the pages and mathematics fix.

None of these re-types the oracle's own formula.  Each check is one of: a value
the pages print (tests/golden), a closed form, a special case that reduces to a
library routine (torch's scaled_dot_product_attention in fp64), an algebraic
identity, an invariant, or a second algorithm the pages describe (the
three-call merge).

Pages cited:
  [BT] "Jet-Long: 具有动态双焦RoPE的高效长上下文扩展" (bittide.aicompass.dev)
  [TW] "NVIDIA研究团队找到了让AI“看清”超长文本的新方法" (techwalker.com)
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "group_size.txt")


def _golden_rows():
    rows = []
    with open(GOLDEN, encoding="utf-8") as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            L, w, G, src = line.split(None, 3)
            rows.append((int(L), int(w), int(G), src))
    return rows


@pytest.mark.parametrize("L,w,G,src", _golden_rows())
def test_group_size_golden(L, w, G, src):
    """[TW] §二/§五/Q1, [BT] §3.1 worked values, plus the workloads' stated G."""
    assert oracle.group_size(L, w) == G, src


def test_group_size_is_smallest_fitting_integer():
    """[BT] §3.1: G is the smallest integer that keeps every remote relative
    position inside the pretrained window.  Checked without the ceil formula:
    the largest remapped distance floor((L-1)/G) - 0 must be <= w - 1 at G and
    (for G > 1) exceed it at G - 1."""
    for L in range(1, 300):
        for w in range(1, 70):
            G = oracle.group_size(L, w)
            assert G >= 1
            assert (L - 1) // G <= w - 1
            if G > 1:
                assert (L - 1) // (G - 1) > w - 1


def test_remap_identity_and_floor():
    """[BT] §3.1: G = 1 gives f(x) = x; f groups G neighbouring positions."""
    for x in range(0, 200):
        assert oracle.remap(x, 1) == x
    for G in (2, 3, 4, 7):
        for x in range(0, 60):
            f = oracle.remap(x, G)
            assert f * G <= x < (f + 1) * G


def test_remote_distance_bound_exhaustive():
    """[BT] §3.1: every remote relative position |f(q) - f(k)| stays within
    w_pretrained.  Exhaustive over all pairs for small L and all w."""
    for L in range(1, 41):
        for w in range(1, L + 1):
            G = oracle.group_size(L, w)
            f = [oracle.remap(x, G) for x in range(L)]
            for i in range(L):
                for j in range(i + 1):
                    assert 0 <= f[i] - f[j] <= w - 1


def test_remote_distance_bound_long():
    """The same bound at long lengths: f is non-decreasing, so the largest
    distance is f(L-1) - f(0)."""
    for w in (1, 2, 3, 128, 4096, 32768):
        for L in list(range(1, 5000, 37)) + [32767, 32768, 32769, 65536, 98304, 131071, 131072]:
            G = oracle.group_size(L, w)
            assert oracle.remap(L - 1, G) - oracle.remap(0, G) <= w - 1


def test_band_definition_points():
    """Local window of exactly w_local keys including the diagonal ([TW] §二);
    causal mask beyond the diagonal."""
    assert oracle.band(10, 11, 4) == 0
    assert oracle.band(10, 10, 4) == 1
    assert oracle.band(10, 7, 4) == 1
    assert oracle.band(10, 6, 4) == 2
    assert oracle.band(10, 10, 0) == 2
    assert oracle.band(10, 0, 4, bifocal=False) == 1


def _rope_complex(x, pos, base):
    """Half-split RoPE written as a complex product: (x_t + i x_{t+h}) e^{i p theta_t}."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    theta = base ** (-2.0 * np.arange(h) / d)
    z = x[..., :h] + 1j * x[..., h:]
    ang = np.asarray(pos, dtype=np.float64).reshape(-1, *([1] * (x.ndim - 1))) * theta
    y = z * np.exp(1j * ang)
    return np.concatenate([y.real, y.imag], axis=-1)


def test_rope_matches_complex_form():
    rng = np.random.default_rng(11)
    for d, base in ((64, 1e4), (128, 1e6), (8, 10.0)):
        x = rng.standard_normal((40, 3, d))
        pos = rng.integers(0, 1 << 17, size=40)
        np.testing.assert_allclose(oracle.rope(x, pos, base), _rope_complex(x, pos, base),
                                   rtol=0, atol=1e-9)


def test_rope_unit_pair_closed_form():
    """d = 2: theta_0 = 1 for any base, so R(p)(1, 0) = (cos p, sin p)."""
    for base in (10.0, 1e4, 1e6):
        pos = np.array([0, 1, 2, 5, 1000, 131071])
        x = np.tile(np.array([[[1.0, 0.0]]]), (len(pos), 1, 1))
        y = oracle.rope(x, pos, base)
        np.testing.assert_allclose(y[:, 0, 0], np.cos(pos), atol=1e-12)
        np.testing.assert_allclose(y[:, 0, 1], np.sin(pos), atol=1e-12)


def test_rotation_composition():
    """[TW] §三: R(a) R(b) = R(a + b), for integer |a|, |b| <= 2^17."""
    rng = np.random.default_rng(3)
    for d, base in ((128, 1e6), (64, 1e4)):
        x = rng.standard_normal((50, 2, d))
        a = rng.integers(-(1 << 17), 1 << 17, size=50)
        b = rng.integers(-(1 << 17), 1 << 17, size=50)
        two = oracle.rope(oracle.rope(x, a, base), b, base)
        one = oracle.rope(x, a + b, base)
        np.testing.assert_allclose(two, one, rtol=0, atol=1e-9)


def test_correction_identity():
    """[BT] §3.3: turning a cached standard-RoPE key R(j) k by f(j) - j gives
    R(f(j)) k; the same holds for the query with f(p) - p."""
    rng = np.random.default_rng(5)
    d, base, G = 128, 1e6, 4
    j = rng.integers(0, 131072, size=64)
    fj = j // G
    k = rng.standard_normal((64, 1, d))
    lhs = oracle.rope(oracle.rope(k, j, base), fj - j, base)
    np.testing.assert_allclose(lhs, oracle.rope(k, fj, base), rtol=0, atol=1e-9)


def _sdpa_plain(q, k, v, scale, base):
    """Plain RoPE causal attention from library routines: complex-form RoPE and
    torch's fp64 scaled_dot_product_attention; LSE from torch.logsumexp."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    pos = np.arange(T)
    qr = torch.from_numpy(_rope_complex(q, pos, base)).permute(1, 0, 2)
    kr = torch.from_numpy(_rope_complex(k, pos, base)).permute(1, 0, 2)
    vv = torch.from_numpy(np.asarray(v, dtype=np.float64)).permute(1, 0, 2)
    kr = kr.repeat_interleave(Hq // Hkv, dim=0)
    vv = vv.repeat_interleave(Hq // Hkv, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(qr[None], kr[None], vv[None],
                                                         is_causal=True, scale=scale)[0]
    s = (qr @ kr.transpose(-1, -2)) * scale
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


@pytest.mark.parametrize("mode", ["G1", "wide_local", "not_bifocal"])
def test_special_cases_equal_plain_attention(mode):
    """[BT] §3.1 / [TW] Q&A Q1: with G = 1 the method is plain RoPE attention.
    Also: a local window covering the sequence, and the bifocal switch off."""
    rng = np.random.default_rng(7)
    T, Hq, Hkv, d, base, scale = 37, 4, 2, 16, 1e4, 0.3
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    kw = dict(rope_base=base, softmax_scale=scale)
    if mode == "G1":
        o, lse = oracle.prefill(q, k, v, w_pretrained=T, w_local=5, **kw)
    elif mode == "wide_local":
        o, lse = oracle.prefill(q, k, v, w_pretrained=4, w_local=T, **kw)
    else:
        o, lse = oracle.prefill(q, k, v, w_pretrained=4, w_local=5, bifocal=False, **kw)
    o_ref, lse_ref = _sdpa_plain(q, k, v, scale, base)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_bifocal_differs_from_plain():
    """Sanity: with G > 1 and a short local window the result is not plain attention."""
    rng = np.random.default_rng(8)
    T, d = 40, 16
    q, k, v = (rng.standard_normal((T, 1, d)) for _ in range(3))
    o, lse = oracle.prefill(q, k, v, w_pretrained=10, w_local=4, rope_base=1e4, softmax_scale=0.5)
    o2, lse2 = _sdpa_plain(q, k, v, 0.5, 1e4)
    assert np.abs(lse - lse2).max() > 1e-2


def test_three_call_merge_equals_direct_form():
    """[TW] §四 and [BT] §3.2: B + A - C, combined with LogSumExp weights, equals
    local keys under standard RoPE and remote keys under remapped RoPE.
    Brute force over small lengths, windows, head dims and GQA."""
    rng = np.random.default_rng(21)
    n = 0
    for L in (1, 2, 5, 17, 48):
        for w_pre in sorted({1, 3, 8, L}):
            for w_local in sorted({0, 1, 2, max(L - 1, 0), L, L + 3}):
                for d, Hq, Hkv in ((2, 1, 1), (8, 4, 2)):
                    q = rng.standard_normal((L, Hq, d))
                    k = rng.standard_normal((L, Hkv, d))
                    v = rng.standard_normal((L, Hkv, d))
                    kw = dict(w_pretrained=w_pre, w_local=w_local, rope_base=100.0,
                              softmax_scale=0.7)
                    o1, l1 = oracle.prefill(q, k, v, **kw)
                    o2, l2 = oracle.prefill_three_call(q, k, v, **kw)
                    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-10)
                    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-10)
                    n += 1
    assert n > 100


def test_zero_query_closed_form():
    """q = 0 makes every score 0 whatever the rotations: O_i is the mean of
    v_0..v_i and LSE_i = ln(i + 1)."""
    rng = np.random.default_rng(2)
    T, Hq, Hkv, d = 33, 2, 1, 8
    q = np.zeros((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    o, lse = oracle.prefill(q, k, v, w_pretrained=8, w_local=5, rope_base=1e4, softmax_scale=1.0)
    mean = np.cumsum(v[:, 0, :], axis=0) / np.arange(1, T + 1)[:, None]
    for h in range(Hq):
        np.testing.assert_allclose(o[:, h, :], mean, atol=1e-13)
        np.testing.assert_allclose(lse[:, h], np.log(np.arange(1, T + 1)), atol=1e-13)


def _probe(i, jstar, L, w_pre, w_local, kappa, d=2, bifocal=1):
    """Boundary probe: q_i = e_0, key j* = kappa e_0, all other keys 0.  Pair 0
    has theta_0 = 1, so the score of j* is kappa cos(distance) with the
    distance i - j* (standard) or f(i) - f(j*) (remapped); every other score is
    0, giving LSE_i = ln(i + exp(kappa cos(distance)))."""
    q = np.zeros((L, 1, d))
    q[:, 0, 0] = 1.0
    k = np.zeros((L, 1, d))
    k[jstar, 0, 0] = kappa
    v = np.zeros((L, 1, d))
    _, lse = oracle.prefill(q, k, v, w_pretrained=w_pre, w_local=w_local, rope_base=1e4,
                            softmax_scale=1.0, rows=[i], bifocal=bifocal)
    return lse[0, 0]


def test_boundary_probe_closed_form():
    """[TW] §二 / [BT] §3.3: the distance i - j = w_local is remote (remapped),
    i - j = w_local - 1 is local (standard).  Chosen so that the two readings
    give LSE values more than 0.05 apart."""
    L, w_pre, w_local, kappa = 64, 16, 7, 3.0
    G = oracle.group_size(L, w_pre)
    assert G == 4
    checked = 0
    for i in range(w_local, L):
        for jstar, expect_remote in ((i - w_local, True), (i - w_local + 1, False)):
            d_std = i - jstar
            d_rem = i // G - jstar // G
            lse_std = math.log(i + math.exp(kappa * math.cos(d_std)))
            lse_rem = math.log(i + math.exp(kappa * math.cos(d_rem)))
            if abs(lse_std - lse_rem) < 0.05:
                continue
            got = _probe(i, jstar, L, w_pre, w_local, kappa)
            want = lse_rem if expect_remote else lse_std
            assert abs(got - want) < 1e-12, (i, jstar)
            checked += 1
    assert checked >= 20


def test_decode_equals_prefill_last_row():
    """[TW] §三 / [BT] §3.3: decode over a cache of standard-RoPE keys, with the
    correction rotation, equals the prefill definition at the last row — for
    every L across the G switch (w_pretrained = 8: G goes 1 -> 2 at L = 9)."""
    rng = np.random.default_rng(13)
    S, Hq, Hkv, d, base, scale = 30, 4, 2, 16, 1e4, 0.4
    q_all = rng.standard_normal((S, Hq, d))
    k = rng.standard_normal((S, Hkv, d))
    v = rng.standard_normal((S, Hkv, d))
    cache_k = oracle.rope(k, np.arange(S), base)  # R(j) k_j, fp64
    for bifocal in (True, False):
        for L in range(1, S + 1):
            kw = dict(w_pretrained=8, w_local=3, rope_base=base, softmax_scale=scale,
                      bifocal=bifocal)
            o_d, lse_d = oracle.decode(q_all[L - 1:L], cache_k[None], v[None], [L], **kw)
            o_p, lse_p = oracle.prefill(q_all[:L], k[:L], v[:L], rows=[L - 1], **kw)
            np.testing.assert_allclose(o_d, o_p, rtol=0, atol=1e-11)
            np.testing.assert_allclose(lse_d, lse_p, rtol=0, atol=1e-11)


def test_decode_batch_is_per_sequence():
    rng = np.random.default_rng(17)
    B, S, Hq, Hkv, d = 3, 20, 2, 1, 8
    q = rng.standard_normal((B, Hq, d))
    kc = rng.standard_normal((B, S, Hkv, d))
    vc = rng.standard_normal((B, S, Hkv, d))
    lens = [20, 7, 13]
    kw = dict(w_pretrained=5, w_local=2, rope_base=1e4, softmax_scale=0.5)
    o, lse = oracle.decode(q, kc, vc, lens, **kw)
    for b in range(B):
        o1, l1 = oracle.decode(q[b:b + 1], kc[b:b + 1], vc[b:b + 1], [lens[b]], **kw)
        np.testing.assert_array_equal(o[b], o1[0])
        np.testing.assert_array_equal(lse[b], l1[0])


def test_varlen_equals_separate_sequences():
    """Packed sequences: each one gets its own G and positions restarting at 0."""
    rng = np.random.default_rng(9)
    lens = [5, 20, 13, 1]
    cu = np.cumsum([0] + lens)
    T, Hq, Hkv, d = int(cu[-1]), 2, 1, 8
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    kw = dict(w_pretrained=6, w_local=3, rope_base=1e4, softmax_scale=0.5)
    o, lse = oracle.prefill(q, k, v, cu_seqlens=cu, **kw)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        o1, l1 = oracle.prefill(q[a:b], k[a:b], v[a:b], **kw)
        np.testing.assert_array_equal(o[a:b], o1)
        np.testing.assert_array_equal(lse[a:b], l1)


def test_row_selection_matches_full():
    rng = np.random.default_rng(4)
    T, d = 25, 8
    q, k, v = (rng.standard_normal((T, 2, d)) for _ in range(3))
    kw = dict(w_pretrained=7, w_local=3, rope_base=1e4, softmax_scale=0.5)
    o, lse = oracle.prefill(q, k, v, **kw)
    rows = [24, 0, 13, 7]
    o2, l2 = oracle.prefill(q, k, v, rows=rows, **kw)
    np.testing.assert_array_equal(o[rows], o2)
    np.testing.assert_array_equal(lse[rows], l2)


def test_bf16_inputs_widen_exactly():
    """bf16 bit patterns are widened exactly: the oracle on bf16 tensors equals
    the oracle on the same values held as fp64."""
    g = torch.Generator().manual_seed(0)
    q = torch.randn(12, 2, 8, generator=g).to(torch.bfloat16)
    k = torch.randn(12, 1, 8, generator=g).to(torch.bfloat16)
    v = torch.randn(12, 1, 8, generator=g).to(torch.bfloat16)
    kw = dict(w_pretrained=4, w_local=2, rope_base=1e4, softmax_scale=0.5)
    o1, l1 = oracle.prefill(q, k, v, **kw)
    o2, l2 = oracle.prefill(q.double(), k.double(), v.double(), **kw)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_chunk_equals_prefill_rows():
    """A prefill chunk over a cache of standard-RoPE keys ([TW] §三, [BT] §3.3)
    equals the prefill definition ([BT] §3.2) at the chunk's rows of the whole
    sequence of length L (G = G(L)), for every L across the G switch
    (w_pretrained = 8: G goes 1 -> 2 at L = 9, 2 -> 3 at L = 17) and several
    chunk sizes, with and without the bifocal split."""
    rng = np.random.default_rng(23)
    S, Hq, Hkv, d, base, scale = 26, 4, 2, 16, 1e4, 0.4
    q_all = rng.standard_normal((S, Hq, d))
    k = rng.standard_normal((S, Hkv, d))
    v = rng.standard_normal((S, Hkv, d))
    cache_k = oracle.rope(k, np.arange(S), base)  # R(j) k_j, fp64
    for bifocal in (True, False):
        kw = dict(w_pretrained=8, w_local=3, rope_base=base, softmax_scale=scale,
                  bifocal=bifocal)
        for L in range(1, S + 1):
            for C in sorted({1, 2, (L + 1) // 2, L}):
                if C > L:
                    continue
                o_c, l_c = oracle.prefill_chunk(q_all[L - C:L], cache_k[None], v[None], [L], **kw)
                o_p, l_p = oracle.prefill(q_all[:L], k[:L], v[:L], rows=range(L - C, L), **kw)
                np.testing.assert_allclose(o_c, o_p, rtol=0, atol=1e-11)
                np.testing.assert_allclose(l_c, l_p, rtol=0, atol=1e-11)


def test_chunk_of_one_is_decode():
    rng = np.random.default_rng(29)
    B, S, Hq, Hkv, d = 2, 40, 4, 2, 8
    q = rng.standard_normal((B, Hq, d))
    kc = rng.standard_normal((B, S, Hkv, d))
    vc = rng.standard_normal((B, S, Hkv, d))
    lens = [40, 17]
    kw = dict(w_pretrained=9, w_local=4, rope_base=1e4, softmax_scale=0.5)
    o_d, l_d = oracle.decode(q, kc, vc, lens, **kw)
    o_c, l_c = oracle.prefill_chunk(q, kc, vc, lens, cu_seqlens_q=[0, 1, 2], **kw)
    np.testing.assert_allclose(o_c, o_d, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_c, l_d, rtol=0, atol=1e-12)


def test_chunk_batch_is_per_sequence():
    """Packed chunks (one of them empty): each sequence gets its own G, its own
    positions and its own cache row; selecting rows changes nothing."""
    rng = np.random.default_rng(31)
    B, S, Hq, Hkv, d = 3, 30, 2, 1, 8
    kc = rng.standard_normal((B, S, Hkv, d))
    vc = rng.standard_normal((B, S, Hkv, d))
    lens, chunks = [30, 11, 19], [7, 0, 19]
    cu = np.cumsum([0] + chunks)
    q = rng.standard_normal((int(cu[-1]), Hq, d))
    kw = dict(w_pretrained=6, w_local=3, rope_base=1e4, softmax_scale=0.5)
    o, lse = oracle.prefill_chunk(q, kc, vc, lens, cu_seqlens_q=cu, **kw)
    for b in range(B):
        a, e = cu[b], cu[b + 1]
        if a == e:
            continue
        o1, l1 = oracle.prefill_chunk(q[a:e], kc[b:b + 1], vc[b:b + 1], [lens[b]], **kw)
        np.testing.assert_array_equal(o[a:e], o1)
        np.testing.assert_array_equal(lse[a:e], l1)
    o_s, l_s = oracle.prefill_chunk(q, kc, vc, lens, cu_seqlens_q=cu, rows=[25, 0, 9], **kw)
    np.testing.assert_array_equal(o_s, o[[25, 0, 9]])
    np.testing.assert_array_equal(l_s, lse[[25, 0, 9]])
    with pytest.raises(ValueError):
        oracle.prefill_chunk(q, kc, vc, [30, 11, 18], cu_seqlens_q=cu, **kw)  # chunk > length


def _hex_rows(name):
    rows = []
    for line in open(os.path.join(os.path.dirname(__file__), "golden", name), encoding="utf-8"):
        line = line.strip()
        if line and not line.startswith("#"):
            a, b, *_ = line.split()
            rows.append((a, b))
    return rows


@pytest.mark.parametrize("code,value", _hex_rows("fp8_e4m3.txt"))
def test_e4m3_values_golden(code, value):
    got = oracle.e4m3_value(int(code, 16))
    if value == "nan":
        assert np.isnan(got)
    else:
        assert got == float(value) and np.signbit(got) == value.startswith("-")


@pytest.mark.parametrize("x,code", _hex_rows("fp8_e4m3_rounding.txt"))
def test_e4m3_rounding_golden(x, code):
    assert oracle.e4m3_encode(float(x)) == int(code, 16)


def test_e4m3_against_torch_float8():
    """Every code's value, and round-to-nearest-even of in-range reals, agree
    with torch's float8_e4m3fn conversions (an independent implementation of
    the same OCP format)."""
    import torch

    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    fin = np.isfinite(ref)
    assert np.array_equal(np.isnan(got), ~fin)
    np.testing.assert_array_equal(got[fin], ref[fin])
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(3000) * 40, rng.standard_normal(1000) * 0.01,
                        (ref[fin][:-1] + ref[fin][1:]) / 2])
    x = np.clip(x, -448, 448).astype(np.float32)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([oracle.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    np.testing.assert_array_equal(mine, t)


def test_e4m3_quant_dequant_roundtrip():
    """Codes survive dequantize -> quantize with the same scale exactly
    (scale a power of two, so value * scale / scale is exact), and the
    quantizer picks the code nearest to x / scale."""
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, size=(5, 3, 8), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x11  # no NaN codes
    scale = np.array([0.25, 1.0, 8.0], dtype=np.float32)
    vals = oracle.e4m3_dequant(codes, scale)
    again = oracle.e4m3_quant(vals.astype(np.float32), scale)
    zero = (codes & 0x7F) == 0
    np.testing.assert_array_equal(again[~zero], codes[~zero])
    x = rng.standard_normal((4, 3, 8)).astype(np.float32) * 30
    q = oracle.e4m3_quant(x, scale)
    back = oracle.e4m3_dequant(q, scale)
    allv = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    for idx in np.ndindex(x.shape):
        t = min(abs(float(x[idx]) / scale[idx[1]]), 448.0)
        assert abs(abs(back[idx]) / scale[idx[1]] - t) <= np.abs(allv - t).min() + 1e-12


def test_decode_fp8_is_decode_of_dequantized_cache():
    """fp8 decode = decode on scale * E4M3(code), the scale per kv head."""
    rng = np.random.default_rng(11)
    B, S, Hq, Hkv, d = 2, 30, 4, 2, 8
    q = rng.standard_normal((B, Hq, d))
    k8 = rng.integers(0, 0x7E, size=(B, S, Hkv, d), dtype=np.uint8)
    v8 = rng.integers(0x80, 0xFE, size=(B, S, Hkv, d), dtype=np.uint8)
    ks, vs = np.array([0.01, 0.02], np.float32), np.array([0.5, 0.25], np.float32)
    kw = dict(w_pretrained=7, w_local=3, rope_base=1e4, softmax_scale=0.5)
    o, lse = oracle.decode_fp8(q, k8, v8, ks, vs, [30, 12], **kw)
    kd = np.vectorize(oracle.e4m3_value)(k8) * ks[None, None, :, None]
    vd = np.vectorize(oracle.e4m3_value)(v8) * vs[None, None, :, None]
    o2, l2 = oracle.decode(q, kd, vd, [30, 12], **kw)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, l2)



# ---- continuous interpolation in the remote window (bifocal = 2) ----------

def test_interp_probe_closed_form():
    """[BT] §4.4 / [TW] §八 variant: a remote pair's angle is (i - j) / s with the
    real scale s = L / w_pretrained (the probe of the boundary test, read off the
    LSE); local pairs keep i - j.  L / w = 2.6 is not an integer, so the angles
    differ from the integer grouping's f(i) - f(j) (G = 3)."""
    L, w_pre, w_local, kappa = 52, 20, 5, 3.0
    s = L / w_pre
    checked = 0
    for i in range(w_local, L):
        for jstar in (0, i // 2, i - w_local, i - w_local + 1, i - 1):
            if jstar < 0 or jstar > i:
                continue
            remote = i - jstar >= w_local
            dist = (i - jstar) / s if remote else i - jstar
            want = math.log(i + math.exp(kappa * math.cos(dist)))
            got = _probe(i, jstar, L, w_pre, w_local, kappa, bifocal=2)
            assert abs(got - want) < 1e-12, (i, jstar)
            checked += 1
    assert checked >= 150


def test_interp_equals_grouping_on_multiples_of_an_integer_scale():
    """When L / w_pretrained is an integer G, x / s = floor(x / G) at multiples
    of G: for a query and a key both at multiples of G the two variants give the
    same remote angle, elsewhere (in general) not."""
    L, w_pre, w_local, kappa = 60, 20, 4, 3.0
    G = oracle.group_size(L, w_pre)
    assert G * w_pre == L
    same = diff = 0
    for i in range(w_local, L):
        for jstar in range(0, i - w_local + 1):
            a = _probe(i, jstar, L, w_pre, w_local, kappa, bifocal=2)
            b = _probe(i, jstar, L, w_pre, w_local, kappa, bifocal=1)
            if i % G == 0 and jstar % G == 0:
                assert abs(a - b) < 1e-12
                same += 1
            elif abs(a - b) > 1e-6:
                diff += 1
    assert same >= 20 and diff >= 100


@pytest.mark.parametrize("L", [10, 20, 21, 33, 47])
def test_interp_short_sequences_and_decode_chunk_paths(L):
    """bifocal = 2: L <= w_pretrained is plain attention (s = 1); decode (the
    correction rotation R(j / s - j) of cache keys) and the chunk form equal the
    prefill definition on the same keys, across s = 1 .. 2.35."""
    rng = np.random.default_rng(L)
    Hq, Hkv, d, base, scale, w_pre, w_local = 4, 2, 16, 1e4, 0.4, 20, 4
    q = rng.standard_normal((L, Hq, d))
    k = rng.standard_normal((L, Hkv, d))
    v = rng.standard_normal((L, Hkv, d))
    kw = dict(w_pretrained=w_pre, w_local=w_local, rope_base=base, softmax_scale=scale)
    o2, l2 = oracle.prefill(q, k, v, bifocal=2, **kw)
    if L <= w_pre:
        o0, l0 = oracle.prefill(q, k, v, bifocal=0, **kw)
        np.testing.assert_allclose(o2, o0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2, l0, rtol=0, atol=1e-12)
    cache = oracle.rope(k, np.arange(L), base)
    od, ld = oracle.decode(q[L - 1:L], cache[None], v[None], [L], bifocal=2, **kw)
    np.testing.assert_allclose(od[0], o2[L - 1], rtol=0, atol=1e-11)
    np.testing.assert_allclose(ld[0], l2[L - 1], rtol=0, atol=1e-11)
    C = (L + 1) // 2
    oc, lc = oracle.prefill_chunk(q[L - C:], cache[None], v[None], [L], bifocal=2, **kw)
    np.testing.assert_allclose(oc, o2[L - C:], rtol=0, atol=1e-11)
    np.testing.assert_allclose(lc, l2[L - C:], rtol=0, atol=1e-11)
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, bifocal=3, **kw)

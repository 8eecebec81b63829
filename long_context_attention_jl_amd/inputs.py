"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module draws random tensors and nothing else: it holds none of the
attention method's arithmetic (no rotation, no remap, no softmax), so both the
HIP path and the CPU oracle can take their inputs from it.

Every tensor comes from ``torch.Generator('cpu').manual_seed(seed)`` and
``torch.randn`` in float32, is scaled, then cast to the working dtype
(bf16 casts round to nearest even).  Draw order is q, then k, then v.

Decode caches are drawn directly as standard-RoPE keys: a rotation maps an
isotropic Gaussian pair to an isotropic Gaussian pair, so i.i.d. N(0, 1) rows
have exactly the distribution of R(j) k_j for raw N(0, 1) keys k_j, and both
sides then read identical cache bits.

Workload shapes follow the pages' evaluation setting: Qwen3-1.7B / Qwen3-8B
attention layers (pretraining window 32768) extended to 65536 and 131072
tokens, local window 2048 ("NVIDIA研究团队找到了让AI“看清”超长文本的新方法",
§二 and §五).  The pages measure on RULER, HELMET-RAG and PG-19; speed depends
only on shapes, so these seeded tensors stand in for those inputs.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch


@dataclasses.dataclass
class Params:
    w_pretrained: int
    w_local: int
    rope_base: float
    softmax_scale: float
    bifocal: bool = True


@dataclasses.dataclass
class PrefillCase:
    name: str
    q: torch.Tensor  # [T, Hq, d] raw (un-rotated), CPU
    k: torch.Tensor  # [T, Hkv, d]
    v: torch.Tensor  # [T, Hkv, d]
    cu_seqlens: Optional[List[int]]
    params: Params

    @property
    def T(self) -> int:
        return self.q.shape[0]

    @property
    def seqlens(self) -> List[int]:
        if self.cu_seqlens is None:
            return [self.T]
        return [b - a for a, b in zip(self.cu_seqlens[:-1], self.cu_seqlens[1:])]


@dataclasses.dataclass
class DecodeCase:
    name: str
    q: torch.Tensor  # [B, Hq, d] raw
    k_cache: torch.Tensor  # [B, S_max, Hkv, d] standard-RoPE keys
    v_cache: torch.Tensor  # [B, S_max, Hkv, d]
    seqlens: List[int]  # L_b: the query sits at position L_b - 1
    params: Params


def _randn(g: torch.Generator, shape, scale: float, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(dtype)


def prefill_inputs(T: int, Hq: int, Hkv: int, d: int, *, seed: int, dtype=torch.bfloat16,
                   q_scale: float = 1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    q = _randn(g, (T, Hq, d), q_scale, dtype)
    k = _randn(g, (T, Hkv, d), 1.0, dtype)
    v = _randn(g, (T, Hkv, d), 1.0, dtype)
    return q, k, v


def decode_inputs(B: int, S_max: int, Hq: int, Hkv: int, d: int, *, seed: int,
                  dtype=torch.bfloat16, q_scale: float = 1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    q = _randn(g, (B, Hq, d), q_scale, dtype)
    k = _randn(g, (B, S_max, Hkv, d), 1.0, dtype)
    v = _randn(g, (B, S_max, Hkv, d), 1.0, dtype)
    return q, k, v


def decode_query(B: int, Hq: int, d: int, *, seed: int, dtype=torch.bfloat16) -> torch.Tensor:
    g = torch.Generator("cpu").manual_seed(seed)
    return _randn(g, (B, Hq, d), 1.0, dtype)


# ---- the five named workloads -------------------------------------------------

def tiny_prefill() -> PrefillCase:
    """1 head, d=64, L=512, w_pretrained=128 (G=4), w_local=32, base 1e4, fp32."""
    q, k, v = prefill_inputs(512, 1, 1, 64, seed=1, dtype=torch.float32)
    return PrefillCase("tiny_f32_L512", q, k, v, None,
                       Params(128, 32, 1e4, 1.0 / math.sqrt(64)))


def qwen3_1p7b_64k() -> PrefillCase:
    """Hq=16, Hkv=8, d=128, L=65536, w_pretrained=32768 (G=2), w_local=2048, base 1e6.
    q is drawn N(0,1) scaled by 1/sqrt(128), which folds the softmax scale into q,
    so the kernel's own scale is 1."""
    q, k, v = prefill_inputs(65536, 16, 8, 128, seed=2, q_scale=1.0 / math.sqrt(128))
    return PrefillCase("qwen3_1p7b_L65536", q, k, v, None, Params(32768, 2048, 1e6, 1.0))


def qwen3_8b_128k() -> PrefillCase:
    """Hq=32, Hkv=8, d=128, L=131072, w_pretrained=32768 (G=4), w_local=2048, base 1e6;
    q scaled by 1/sqrt(128) (softmax scale 1)."""
    q, k, v = prefill_inputs(131072, 32, 8, 128, seed=3, q_scale=1.0 / math.sqrt(128))
    return PrefillCase("qwen3_8b_L131072", q, k, v, None, Params(32768, 2048, 1e6, 1.0))


def varlen_4seq() -> PrefillCase:
    """Four packed sequences of 8192, 32768, 49152, 98304 tokens (G = 1, 1, 2, 3),
    Hq=32, Hkv=8, d=128, w_pretrained=32768, w_local=2048, base 1e6, scale 1/sqrt(128)."""
    lens = [8192, 32768, 49152, 98304]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    q, k, v = prefill_inputs(cu[-1], 32, 8, 128, seed=5)
    return PrefillCase("varlen_4seq_T188416", q, k, v, cu,
                       Params(32768, 2048, 1e6, 1.0 / math.sqrt(128)))


DECODE_PARAMS = Params(32768, 2048, 1e6, 1.0 / math.sqrt(128))


def decode_128k() -> DecodeCase:
    """One new query (32 q heads, 8 kv heads, d=128) against a cache of 131071
    keys plus the appended current token: L = 131072, G = 4."""
    q, k, v = decode_inputs(1, 131072, 32, 8, 128, seed=4)
    return DecodeCase("decode_L131072", q, k, v, [131072], DECODE_PARAMS)


def decode_16step_cache():
    """Cache for 16 consecutive decode steps: rows 0..32775 (the cache filled to
    32760 plus the 16 appended tokens).  Step s (0-based) attends L = 32761 + s
    keys, so L crosses 32768 -> 32769 (G 1 -> 2) between steps 7 and 8."""
    g = torch.Generator("cpu").manual_seed(4 + 1000)
    S_max = 32776
    k = _randn(g, (1, S_max, 8, 128), 1.0, torch.bfloat16)
    v = _randn(g, (1, S_max, 8, 128), 1.0, torch.bfloat16)
    lens = [32761 + s for s in range(16)]
    queries = [decode_query(1, 32, 128, seed=4 + 100 * (s + 1)) for s in range(16)]
    return queries, k, v, lens, DECODE_PARAMS


@dataclasses.dataclass
class ChunkCase:
    name: str
    q: torch.Tensor  # [Tq, Hq, d] raw: the chunks' new rows, packed
    k_cache: torch.Tensor  # [B, S_max, Hkv, d] standard-RoPE keys (the chunks' own included)
    v_cache: torch.Tensor  # [B, S_max, Hkv, d]
    seqlens: List[int]  # L_b: keys of sequence b; its chunk is positions L_b - C_b .. L_b - 1
    cu_q: Optional[List[int]]  # chunk offsets in q (None: one chunk)
    params: Params


def chunk_inputs(chunks: List[int], seqlens: List[int], S_max: int, Hq: int, Hkv: int, d: int,
                 *, seed: int, dtype=torch.bfloat16):
    """Packed chunk queries [sum(chunks), Hq, d] and caches [B, S_max, Hkv, d]."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = _randn(g, (sum(chunks), Hq, d), 1.0, dtype)
    k = _randn(g, (len(seqlens), S_max, Hkv, d), 1.0, dtype)
    v = _randn(g, (len(seqlens), S_max, Hkv, d), 1.0, dtype)
    cu = [0]
    for c in chunks:
        cu.append(cu[-1] + c)
    return q, k, v, cu


def chunk_128k() -> ChunkCase:
    """A chunk of 4096 new rows (32 q heads, 8 kv heads, d=128) appended to a
    cache of 126976 keys: the chunk is positions 126976 .. 131071 of a sequence
    of L = 131072 (G = 4), w_local 2048."""
    q, k, v, _ = chunk_inputs([4096], [131072], 131072, 32, 8, 128, seed=6)
    return ChunkCase("chunk4096_L131072", q, k, v, [131072], None, DECODE_PARAMS)


def to_e4m3(x: torch.Tensor):
    """Stores a [..., H, d] cache block as OCP E4M3 codes with one scale per head
    (scale = max |x| of the head / 448, so every value is in range), using
    torch's own float8_e4m3fn conversion.  Returns (uint8 codes, float32 scales)."""
    xf = x.float()
    H = xf.shape[-2]
    amax = xf.abs().transpose(0, -2).reshape(H, -1).amax(dim=1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    codes = (xf / scale.view(H, 1)).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def decode_fp8_inputs(B: int, S_max: int, Hq: int, Hkv: int, d: int, *, seed: int):
    """bf16 queries and an fp8 cache: the bf16 caches of ``decode_inputs``
    stored as E4M3 codes with per-kv-head scales."""
    q, k, v = decode_inputs(B, S_max, Hq, Hkv, d, seed=seed)
    k8, ks = to_e4m3(k)
    v8, vs = to_e4m3(v)
    return q, k8, v8, ks, vs


def decode_fp8_128k():
    """The 128K decode workload (L = 131072, G = 4) on an fp8 cache."""
    q, k8, v8, ks, vs = decode_fp8_inputs(1, 131072, 32, 8, 128, seed=4)
    return q, k8, v8, ks, vs, [131072], DECODE_PARAMS


def outlier_value_channels(d: int):
    """The value channels with_outlier_channels makes large (by default)."""
    return (10, d - 28)


def with_outlier_channels(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, seed: int,
                          k_channels=(3,), v_channels=None, k_range=(1.0e3, 3.0e4),
                          v_range=(1.0e3, 6.0e4), q_small: float = 7.0e-5):
    """Large-magnitude variant of seeded inputs (any shape whose last dim is d).

    Every key gets, in each channel of ``k_channels``, a value of random sign
    and magnitude uniform in ``k_range``; every value gets the same in each
    channel of ``v_channels`` with ``v_range``.  The query channels c and
    c + d/2 of each key channel c (the two channels a half-split RoPE pair
    mixes) are redrawn as N(0, 1) * q_small, so the scores stay of order one
    while the keys reach ``k_range[1]``.  Everything else is left as drawn.
    Returns new tensors of the inputs' dtype (bf16 rounds to nearest even)."""
    g = torch.Generator("cpu").manual_seed(seed)
    d = q.shape[-1]
    if v_channels is None:
        v_channels = outlier_value_channels(d)
    q, k, v = q.float().clone(), k.float().clone(), v.float().clone()

    def big(shape, lo, hi):
        mag = lo + (hi - lo) * torch.rand(*shape, generator=g, dtype=torch.float32)
        sign = torch.where(torch.rand(*shape, generator=g) < 0.5, -1.0, 1.0)
        return mag * sign

    for c in k_channels:
        k[..., c] = big(k.shape[:-1], *k_range)
        for cq in (c, (c + d // 2) % d):
            q[..., cq] = torch.randn(*q.shape[:-1], generator=g, dtype=torch.float32) * q_small
    for c in v_channels:
        v[..., c] = big(v.shape[:-1], *v_range)
    return q, k, v


def sink_channels(d: int, n_pairs: int = 4):
    """The RoPE channels of the n_pairs lowest-frequency pairs (t, t + d/2),
    t = d/2 - n_pairs .. d/2 - 1: their angles stay small at every position
    of the workloads, so a score through them hardly depends on position."""
    half = d // 2
    return [t for t in range(half - n_pairs, half)] + [t + half for t in range(half - n_pairs, half)]


def with_sink_key(q: torch.Tensor, k: torch.Tensor, *, first_keys, q_add: float, k_value: float,
                  n_pairs: int = 4):
    """Attention-sink variant of seeded inputs: every query gets q_add added in
    the sink channels (sink_channels(d, n_pairs)), and the keys at the rows in
    first_keys (the first key of each sequence, or of a cache) get k_value in
    those channels, every head.  Each query then scores that key about
    2 n_pairs q_add k_value (times the softmax scale) above its other keys,
    whatever its position: one key carries most of every softmax.  Returns
    new float32 tensors (q's and k's shapes)."""
    q = q.float().clone()
    k = k.float().clone()
    ch = sink_channels(q.shape[-1], n_pairs)
    q[..., ch] += q_add
    for r in first_keys:
        k[r][..., ch] = k_value
    return q, k


def to_dtype(dtype, *ts):
    return tuple(t.to(dtype) for t in ts)

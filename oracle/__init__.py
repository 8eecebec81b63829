"""fp64 CPU oracle for Dynamic Bifocal RoPE attention (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library under
``long_context_attention_jl_amd`` never does, and shares no code with it.

The arithmetic lives in ``jl_oracle.c`` (plain C, fp64, OpenMP over rows);
this module only builds it with gcc and marshals numpy arrays.  Each function
cites the page section it follows; see the header of ``jl_oracle.c`` for the
readings taken where the pages are silent.

Pages cited:
  [BT] "Jet-Long: 具有动态双焦RoPE的高效长上下文扩展" (bittide.aicompass.dev)
  [TW] "NVIDIA研究团队找到了让AI“看清”超长文本的新方法" (techwalker.com)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "jl_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, F64 = 0, 1, 2

_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)
_vp = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile jl_oracle.c with gcc (fp64, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.jlo_group_size.restype = ctypes.c_int64
        lib.jlo_group_size.argtypes = [ctypes.c_int64, ctypes.c_int64]
        lib.jlo_remap.restype = ctypes.c_int64
        lib.jlo_remap.argtypes = [ctypes.c_int64, ctypes.c_int64]
        lib.jlo_band.restype = ctypes.c_int
        lib.jlo_band.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
        lib.jlo_rope.restype = None
        lib.jlo_rope.argtypes = [_f64p, _vp, ctypes.c_int, _i64p, ctypes.c_int64, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_double]
        common = [_vp, _vp, _vp, ctypes.c_int, _i64p, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                  ctypes.c_double]
        lib.jlo_prefill.restype = ctypes.c_int
        lib.jlo_prefill.argtypes = [_f64p, _f64p] + common + [ctypes.c_int, _i64p, ctypes.c_int64,
                                                            ctypes.c_int]
        lib.jlo_prefill_three_call.restype = ctypes.c_int
        lib.jlo_prefill_three_call.argtypes = [_f64p, _f64p] + common + [_i64p, ctypes.c_int64]
        lib.jlo_decode.restype = ctypes.c_int
        lib.jlo_decode.argtypes = [_f64p, _f64p, _vp, _vp, _vp, ctypes.c_int, _i64p, ctypes.c_int,
                                   ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                   ctypes.c_double, ctypes.c_int, ctypes.c_int]
        lib.jlo_prefill_chunk.restype = ctypes.c_int
        lib.jlo_prefill_chunk.argtypes = [_f64p, _f64p, _vp, _vp, _vp, ctypes.c_int, _i64p, _i64p,
                                          ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                          ctypes.c_double, ctypes.c_int, _i64p, ctypes.c_int64,
                                          ctypes.c_int]
        lib.jlo_e4m3_value.restype = ctypes.c_double
        lib.jlo_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.jlo_e4m3_encode.restype = ctypes.c_uint8
        lib.jlo_e4m3_encode.argtypes = [ctypes.c_double]
        lib.jlo_e4m3_dequant.restype = None
        lib.jlo_e4m3_dequant.argtypes = [_f64p, _vp, _vp, ctypes.c_int64, ctypes.c_int,
                                         ctypes.c_int]
        lib.jlo_e4m3_quant.restype = None
        lib.jlo_e4m3_quant.argtypes = [_vp, _vp, ctypes.c_int, _vp, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_int]
        _lib = lib
    return _lib


def _host(a):
    """Return (contiguous numpy array, dtype code).  Accepts numpy arrays or CPU
    torch tensors (bf16 tensors are passed as their raw 16-bit patterns)."""
    try:
        import torch

        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                return a.view(torch.int16).numpy().view(np.uint16), BF16
            if a.dtype == torch.float32:
                return a.numpy(), F32
            if a.dtype == torch.float64:
                return a.numpy(), F64
            raise TypeError("unsupported tensor dtype %s" % a.dtype)
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.float64:
        return a, F64
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError("unsupported array dtype %s" % a.dtype)


def _ptr(a, t=None):
    if t is None:
        return ctypes.c_void_p(a.ctypes.data)
    return a.ctypes.data_as(t)


def group_size(L: int, w_pretrained: int) -> int:
    """[BT] §3.1: G = max(1, ceil(L / w_pretrained))."""
    return int(_load().jlo_group_size(int(L), int(w_pretrained)))


def remap(x: int, G: int) -> int:
    """[BT] §3.1: f(x) = floor(x / G)."""
    return int(_load().jlo_remap(int(x), int(G)))


def band(i: int, j: int, w_local: int, bifocal: bool = True) -> int:
    """0 masked (j > i), 1 local (0 <= i-j < w_local), 2 remote.  [TW] §二, [BT] §3.3."""
    return int(_load().jlo_band(int(i), int(j), int(w_local), _mode(bifocal)))


def rope(x, positions, rope_base: float) -> np.ndarray:
    """fp64 half-split RoPE: out[t, h] = R(positions[t]) x[t, h]; x is [T, H, d]."""
    xa, dt = _host(x)
    T, H, d = xa.shape
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64).reshape(T))
    out = np.empty((T, H, d), dtype=np.float64)
    _load().jlo_rope(_ptr(out, _f64p), _ptr(xa), dt, _ptr(pos, _i64p), T, H, d, float(rope_base))
    return out


def _mode(bifocal) -> int:
    """0 plain RoPE, 1 the method (integer grouping), 2 continuous interpolation
    in the remote window; booleans map to 0 and 1."""
    m = int(bifocal)
    if m not in (0, 1, 2):
        raise ValueError("bifocal must be 0, 1 or 2")
    return m


def _cu(cu_seqlens, T):
    if cu_seqlens is None:
        return np.array([0, T], dtype=np.int64)
    return np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))


def prefill(q, k, v, *, w_pretrained, w_local, rope_base, softmax_scale, bifocal=True,
            cu_seqlens=None, rows=None, n_threads=0):
    """Direct definition of bifocal causal prefill ([BT] §3.2).

    q [T, Hq, d], k/v [T, Hkv, d] (raw, un-rotated).  Returns (o, lse) in fp64
    with o [R, Hq, d] and lse [R, Hq] for the R selected rows (all rows when
    ``rows`` is None).
    """
    qa, dt = _host(q)
    ka, dk = _host(k)
    va, dv = _host(v)
    assert dt == dk == dv, "q, k, v must share one dtype"
    T, Hq, d = qa.shape
    Hkv = ka.shape[1]
    cu = _cu(cu_seqlens, T)
    if rows is None:
        R, rp = T, None
    else:
        ra = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        R, rp = len(ra), _ptr(ra, _i64p)
    o = np.empty((R, Hq, d), dtype=np.float64)
    lse = np.empty((R, Hq), dtype=np.float64)
    rc = _load().jlo_prefill(_ptr(o, _f64p), _ptr(lse, _f64p), _ptr(qa), _ptr(ka), _ptr(va), dt,
                             _ptr(cu, _i64p), len(cu) - 1, T, Hq, Hkv, d, int(w_pretrained),
                             int(w_local), float(rope_base), float(softmax_scale),
                             _mode(bifocal), rp, R, int(n_threads))
    if rc != 0:
        raise ValueError("oracle prefill rejected its arguments")
    return o, lse


def prefill_three_call(q, k, v, *, w_pretrained, w_local, rope_base, softmax_scale,
                       cu_seqlens=None, rows=None):
    """The pages' three-call form (B + A - C merged in LSE space; [TW] §四, [BT] §3.2)."""
    qa, dt = _host(q)
    ka, _ = _host(k)
    va, _ = _host(v)
    T, Hq, d = qa.shape
    Hkv = ka.shape[1]
    cu = _cu(cu_seqlens, T)
    if rows is None:
        R, rp = T, None
    else:
        ra = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        R, rp = len(ra), _ptr(ra, _i64p)
    o = np.empty((R, Hq, d), dtype=np.float64)
    lse = np.empty((R, Hq), dtype=np.float64)
    rc = _load().jlo_prefill_three_call(_ptr(o, _f64p), _ptr(lse, _f64p), _ptr(qa), _ptr(ka),
                                        _ptr(va), dt, _ptr(cu, _i64p), len(cu) - 1, T, Hq, Hkv, d,
                                        int(w_pretrained), int(w_local), float(rope_base),
                                        float(softmax_scale), rp, R)
    if rc != 0:
        raise ValueError("oracle three-call prefill rejected its arguments")
    return o, lse


def decode(q, k_cache, v_cache, seqlens, *, w_pretrained, w_local, rope_base, softmax_scale,
           bifocal=True, n_threads=0):
    """Decode with the on-the-fly correction rotation ([TW] §三, [BT] §3.3).

    q [B, Hq, d] raw; k_cache/v_cache [B, S_max, Hkv, d] holding standard-RoPE
    keys at their original positions; seqlens[b] = L_b (query at L_b - 1).
    Returns (o [B, Hq, d], lse [B, Hq]) in fp64.
    """
    qa, dt = _host(q)
    ka, dk = _host(k_cache)
    va, dv = _host(v_cache)
    assert dt == dk == dv
    B, Hq, d = qa.shape
    S_max, Hkv = ka.shape[1], ka.shape[2]
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int64).reshape(B))
    o = np.empty((B, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    rc = _load().jlo_decode(_ptr(o, _f64p), _ptr(lse, _f64p), _ptr(qa), _ptr(ka), _ptr(va), dt,
                            _ptr(sl, _i64p), B, S_max, Hq, Hkv, d, int(w_pretrained), int(w_local),
                            float(rope_base), float(softmax_scale), _mode(bifocal),
                            int(n_threads))
    if rc != 0:
        raise ValueError("oracle decode rejected its arguments")
    return o, lse


def prefill_chunk(q, k_cache, v_cache, seqlens, *, w_pretrained, w_local, rope_base,
                  softmax_scale, bifocal=True, cu_seqlens_q=None, rows=None, n_threads=0):
    """A prefill chunk against a cache ([TW] §三, [BT] §3.1, §3.3).

    q [Tq, Hq, d] raw: the newest C_b positions L_b - C_b .. L_b - 1 of each
    sequence b, packed by ``cu_seqlens_q`` (None: one sequence, C = Tq);
    k_cache/v_cache [B, S_max, Hkv, d] hold the L_b = seqlens[b] keys of the
    sequence (standard-RoPE keys at their original positions, the chunk's own
    keys included).  G = G(L_b).  Returns (o [R, Hq, d], lse [R, Hq]) in fp64
    for the R selected rows of q (all when ``rows`` is None).
    """
    qa, dt = _host(q)
    ka, dk = _host(k_cache)
    va, dv = _host(v_cache)
    assert dt == dk == dv
    Tq, Hq, d = qa.shape
    B, S_max, Hkv = ka.shape[0], ka.shape[1], ka.shape[2]
    cu = _cu(cu_seqlens_q, Tq)
    assert len(cu) == B + 1, "one chunk per cache row"
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int64).reshape(B))
    if rows is None:
        R, rp = Tq, None
    else:
        ra = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        R, rp = len(ra), _ptr(ra, _i64p)
    o = np.empty((R, Hq, d), dtype=np.float64)
    lse = np.empty((R, Hq), dtype=np.float64)
    rc = _load().jlo_prefill_chunk(_ptr(o, _f64p), _ptr(lse, _f64p), _ptr(qa), _ptr(ka),
                                   _ptr(va), dt, _ptr(cu, _i64p), _ptr(sl, _i64p), B, Tq, S_max,
                                   Hq, Hkv, d, int(w_pretrained), int(w_local), float(rope_base),
                                   float(softmax_scale), _mode(bifocal), rp, R,
                                   int(n_threads))
    if rc != 0:
        raise ValueError("oracle chunked prefill rejected its arguments")
    return o, lse


# ---- fp8 (OCP E4M3) KV cache ------------------------------------------------

def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3 code (bias 7, subnormals, S.1111.111 = NaN)."""
    return float(_load().jlo_e4m3_value(int(code)))


def e4m3_encode(x: float) -> int:
    """Nearest E4M3 code, ties to even, saturating at +-448."""
    return int(_load().jlo_e4m3_encode(float(x)))


def _codes(a):
    try:
        import torch

        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous().view(torch.uint8).numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint8, "fp8 caches are passed as their uint8 codes"
    return a


def e4m3_dequant(codes, scale) -> np.ndarray:
    """fp64 values scale[h] * E4M3(code) of a [..., H, d] cache."""
    c = _codes(codes)
    H, d = c.shape[-2], c.shape[-1]
    sc = np.ascontiguousarray(np.asarray(scale, dtype=np.float32).reshape(H))
    out = np.empty(c.shape, dtype=np.float64)
    _load().jlo_e4m3_dequant(_ptr(out, _f64p), _ptr(c), _ptr(sc), c.size // (H * d), H, d)
    return out


def e4m3_quant(x, scale) -> np.ndarray:
    """E4M3 codes of x / scale[h] for a [..., H, d] cache (fp32 quotient, RNE,
    saturating); returns uint8 of x's shape."""
    xa, dt = _host(x)
    H, d = xa.shape[-2], xa.shape[-1]
    sc = np.ascontiguousarray(np.asarray(scale, dtype=np.float32).reshape(H))
    out = np.empty(xa.shape, dtype=np.uint8)
    _load().jlo_e4m3_quant(_ptr(out), _ptr(xa), dt, _ptr(sc), xa.size // (H * d), H, d)
    return out


def decode_fp8(q, k_codes, v_codes, k_scale, v_scale, seqlens, **kw):
    """Bifocal decode ([TW] §三, [BT] §3.3) on an fp8 cache: the keys and values
    are scale[h] * E4M3(code); the rest is ``decode`` on those fp64 values."""
    kc = e4m3_dequant(k_codes, k_scale)
    vc = e4m3_dequant(v_codes, v_scale)
    qa, _ = _host(q)
    if qa.dtype == np.uint16:  # bf16 bits -> fp64, exact
        qa = (qa.astype(np.uint32) << 16).view(np.float32)
    return decode(qa.astype(np.float64), kc, vc, seqlens, **kw)

"""ctypes binding of libjetlong (argument marshalling only).

Every step of the computation runs in the HIP kernels of ``libjetlong.so``;
this module converts torch tensors to pointers, allocates outputs and the
workspace with torch (device memory plumbing) and passes the caller's current
HIP stream.  There is no fallback: if the library is missing or a call fails,
an exception is raised.

Pages cited:
  [BT] "Jet-Long: 具有动态双焦RoPE的高效长上下文扩展" (bittide.aicompass.dev)
  [TW] "NVIDIA研究团队找到了让AI“看清”超长文本的新方法" (techwalker.com)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjetlong.so")

JL_OK = 0
JL_ERR_INVALID_ARGUMENT = 1
JL_ERR_UNSUPPORTED = 2
JL_ERR_WORKSPACE_TOO_SMALL = 3
JL_ERR_HIP = 4
JL_DTYPE_F32 = 0
JL_DTYPE_BF16 = 1


class JLError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__("%s failed: %s (%s)" % (fn, _STATUS.get(status, status), msg))
        self.status = status


_STATUS = {0: "JL_OK", 1: "JL_ERR_INVALID_ARGUMENT", 2: "JL_ERR_UNSUPPORTED",
           3: "JL_ERR_WORKSPACE_TOO_SMALL", 4: "JL_ERR_HIP"}


class jl_params(ctypes.Structure):
    _fields_ = [("w_pretrained", ctypes.c_int32), ("w_local", ctypes.c_int32),
                ("rope_base", ctypes.c_double), ("softmax_scale", ctypes.c_float),
                ("bifocal", ctypes.c_int32), ("precise", ctypes.c_int32),
                ("reuse_images", ctypes.c_int32)]


_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


def lib() -> ctypes.CDLL:
    """Load libjetlong.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libjetlong.so is not built; run __graft_entry__.build() "
                               "or python long_context_attention_jl_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        L.jl_abi_version.restype = ctypes.c_int
        L.jl_status_string.restype = ctypes.c_char_p
        L.jl_status_string.argtypes = [ctypes.c_int]
        L.jl_last_error.restype = ctypes.c_char_p
        L.jl_group_size.restype = ctypes.c_int
        L.jl_group_size.argtypes = [_i64, _i32, ctypes.POINTER(_i32)]
        L.jl_rope_apply.restype = ctypes.c_int
        L.jl_rope_apply.argtypes = [_vp, _vp, _vp, _i64, _i32, _i32, ctypes.c_double, _i32, ctypes.c_int, _vp]
        L.jl_bifocal_prefill_workspace.restype = ctypes.c_int
        L.jl_bifocal_prefill_workspace.argtypes = [_i64, _i32, _i32, _i32, _i32, ctypes.c_int,
                                                   ctypes.POINTER(jl_params),
                                                   ctypes.POINTER(ctypes.c_size_t)]
        L.jl_bifocal_prefill.restype = ctypes.c_int
        L.jl_bifocal_prefill.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32,
                                         _i32, ctypes.POINTER(jl_params), ctypes.c_int, _vp, _vp,
                                         ctypes.c_size_t, _vp]
        L.jl_bifocal_prefill_three_call_workspace.restype = ctypes.c_int
        L.jl_bifocal_prefill_three_call_workspace.argtypes = [_i64, _i32, _i32, _i32, _i32,
                                                              ctypes.c_int,
                                                              ctypes.POINTER(jl_params),
                                                              ctypes.POINTER(ctypes.c_size_t)]
        L.jl_bifocal_prefill_three_call.restype = ctypes.c_int
        L.jl_bifocal_prefill_three_call.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32,
                                                    _i32, _i32, _i32, ctypes.POINTER(jl_params),
                                                    ctypes.c_int, _vp, ctypes.c_size_t, _vp]
        L.jl_bifocal_decode_workspace.restype = ctypes.c_int
        L.jl_bifocal_decode_workspace.argtypes = [_i32, _i32, _i32, _i32, _i32, ctypes.c_int,
                                                  ctypes.POINTER(ctypes.c_size_t)]
        L.jl_bifocal_decode.restype = ctypes.c_int
        L.jl_bifocal_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _i32, _i32,
                                        _i32, ctypes.POINTER(jl_params), ctypes.c_int, _vp,
                                        ctypes.c_size_t, _vp]
        L.jl_bifocal_decode_noalloc.restype = ctypes.c_int
        L.jl_bifocal_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64,
                                                _i32, _i32, _i32, ctypes.POINTER(jl_params),
                                                ctypes.c_int, _vp]
        L.jl_bifocal_decode_three_call_workspace.restype = ctypes.c_int
        L.jl_bifocal_decode_three_call_workspace.argtypes = [_i32, _i32, _i32, _i32, _i32,
                                                             ctypes.c_int,
                                                             ctypes.POINTER(jl_params),
                                                             ctypes.POINTER(ctypes.c_size_t)]
        L.jl_bifocal_decode_three_call.restype = ctypes.c_int
        L.jl_bifocal_decode_three_call.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64,
                                                   _i32, _i32, _i32, ctypes.POINTER(jl_params),
                                                   ctypes.c_int, _vp, ctypes.c_size_t, _vp]
        L.jl_bifocal_decode_paged.restype = ctypes.c_int
        L.jl_bifocal_decode_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                              _i64, _i32, _i32, _i32, _i32,
                                              ctypes.POINTER(jl_params), ctypes.c_int, _vp,
                                              ctypes.c_size_t, _vp]
        L.jl_bifocal_prefill_chunk_workspace.restype = ctypes.c_int
        L.jl_bifocal_prefill_chunk_workspace.argtypes = [_i64, _i32, _i32, _i32, _i32, _i32,
                                                         ctypes.c_int, ctypes.POINTER(jl_params),
                                                         ctypes.POINTER(ctypes.c_size_t)]
        L.jl_bifocal_prefill_chunk.restype = ctypes.c_int
        L.jl_bifocal_prefill_chunk.argtypes = [_vp, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _vp,
                                               _i32, _i32, _i64, _i32, _i32, _i32,
                                               ctypes.POINTER(jl_params), ctypes.c_int, _vp,
                                               ctypes.c_size_t, _vp]
        L.jl_bifocal_prefill_chunk_paged.restype = ctypes.c_int
        L.jl_bifocal_prefill_chunk_paged.argtypes = [_vp, _vp, _vp, _vp, _i64, _i32, _vp, _vp,
                                                     _vp, _vp, _i32, _i32, _i32, _i64, _i32,
                                                     _i32, _i32, _i32, ctypes.POINTER(jl_params),
                                                     ctypes.c_int, _vp, ctypes.c_size_t, _vp]
        L.jl_bifocal_decode_fp8.restype = ctypes.c_int
        L.jl_bifocal_decode_fp8.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                            _i64, _i32, _i32, _i32, ctypes.POINTER(jl_params),
                                            _vp, ctypes.c_size_t, _vp]
        L.jl_bifocal_decode_fp8_paged.restype = ctypes.c_int
        L.jl_bifocal_decode_fp8_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                  _i32, _i32, _i32, _i64, _i32, _i32, _i32, _i32,
                                                  ctypes.POINTER(jl_params), _vp,
                                                  ctypes.c_size_t, _vp]
        L.jl_kv_quantize_fp8.restype = ctypes.c_int
        L.jl_kv_quantize_fp8.argtypes = [_vp, _vp, _vp, _i64, _i32, _i32, _vp]
        L.jl_debug_index_math.restype = ctypes.c_int
        L.jl_debug_index_math.argtypes = [_i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]
        L.jl_debug_stream_read.restype = ctypes.c_int
        L.jl_debug_stream_read.argtypes = [_vp, ctypes.c_size_t, _vp, _vp]
        L.jl_debug_mfma_stream.restype = ctypes.c_int
        L.jl_debug_mfma_stream.argtypes = [_vp, ctypes.c_size_t, _i32, _vp, _vp]
        L.jl_profile_enable.restype = ctypes.c_int
        L.jl_profile_enable.argtypes = [_i32]
        L.jl_profile_read.restype = ctypes.c_int
        L.jl_profile_read.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(_i32),
                                      ctypes.POINTER(ctypes.c_double), _i32, ctypes.POINTER(_i32)]
        _lib = L
    return _lib


def _check(st: int, fn: str) -> None:
    if st != JL_OK:
        msg = lib().jl_last_error()
        raise JLError(st, fn, msg.decode() if msg else "")


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return JL_DTYPE_BF16
    if t.dtype == torch.float32:
        return JL_DTYPE_F32
    raise TypeError("libjetlong takes bfloat16 or float32 tensors, got %s" % t.dtype)


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _expect(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _like(t: Optional[torch.Tensor], name: str, shape, dtype, device) -> None:
    """An optional caller-supplied tensor must have exactly this shape, dtype
    and device (the library writes or reads exactly that many elements)."""
    if t is None:
        return
    _expect(tuple(t.shape) == tuple(shape), "%s must have shape %s, got %s"
            % (name, tuple(shape), tuple(t.shape)))
    _expect(t.dtype == dtype, "%s must be %s, got %s" % (name, dtype, t.dtype))
    _expect(t.device == device, "%s must be on %s, got %s" % (name, device, t.device))


def _rank(t: torch.Tensor, name: str, n: int) -> None:
    _expect(t.dim() == n, "%s must have %d dimensions, got shape %s" % (name, n, tuple(t.shape)))


def _check_qkv(q, k, v, out, lse_out, k_rot_out=None):
    """Prefill operands: q [T, Hq, d]; k, v [T, Hkv, d] of q's dtype and device."""
    _rank(q, "q", 3)
    _rank(k, "k", 3)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    _expect(q.dtype in (torch.bfloat16, torch.float32), "q must be bfloat16 or float32")
    _expect(k.shape[0] == T and k.shape[2] == d, "k must be [T, Hkv, d] = [%d, Hkv, %d], got %s"
            % (T, d, tuple(k.shape)))
    _like(k, "k", (T, Hkv, d), q.dtype, q.device)
    _like(v, "v", (T, Hkv, d), q.dtype, q.device)
    _like(out, "out", (T, Hq, d), q.dtype, q.device)
    _like(lse_out, "lse_out", (Hq, T), torch.float32, q.device)
    _like(k_rot_out, "k_rot_out", (T, Hkv, d), q.dtype, q.device)


def _check_cache(q, k_cache, v_cache, out, lse_out, *, batch_dim: bool, cache_dtype=None):
    """Decode / chunk operands: caches [B', S, Hkv, d] (B' >= batch when batch_dim)
    or page pools [n_pages, page_size, Hkv, d]; values like keys."""
    _rank(q, "q", 3)
    _rank(k_cache, "k_cache", 4)
    Bq, Hq, d = q.shape
    _expect(q.dtype in (torch.bfloat16, torch.float32), "q must be bfloat16 or float32")
    _expect(k_cache.shape[3] == d, "the caches' last dimension must be d = %d, got %s"
            % (d, tuple(k_cache.shape)))
    cdt = q.dtype if cache_dtype is None else k_cache.dtype
    if cache_dtype is not None:
        _expect(k_cache.dtype in cache_dtype, "k_cache must be one of %s" % (cache_dtype,))
    _like(k_cache, "k_cache", tuple(k_cache.shape), cdt, q.device)
    _like(v_cache, "v_cache", tuple(k_cache.shape), cdt, q.device)
    _like(out, "out", tuple(q.shape), q.dtype, q.device)
    _expect(k_cache.shape[2] >= 1 and Hq % k_cache.shape[2] == 0,
            "Hq = %d must be a multiple of the caches' kv heads %d" % (Hq, k_cache.shape[2]))
    return Bq, Hq, d


def _check_lens(n: int, batch: int, name: str) -> None:
    _expect(n == batch, "%s needs one entry per sequence (%d), got %d" % (name, batch, n))


def _check_block_table(bt: torch.Tensor, batch: int, device) -> None:
    _rank(bt, "block_table", 2)
    _expect(bt.shape[0] >= batch, "block_table needs a row per sequence (%d), got %d"
            % (batch, bt.shape[0]))
    _expect(bt.device == device, "block_table must be on %s" % device)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _params(w_pretrained, w_local, rope_base, softmax_scale, bifocal, precise=False,
            reuse_images=False) -> jl_params:
    """bifocal: False / 0 plain RoPE, True / 1 the method (integer grouping in the
    remote window), 2 continuous interpolation in the remote window.
    precise: split-precision scores (for concentrated attention).
    reuse_images: chunk calls keep the key/value images of earlier calls on
    the same workspace while they hold."""
    return jl_params(int(w_pretrained), int(w_local), float(rope_base), float(softmax_scale),
                     int(bifocal), 1 if precise else 0, 1 if reuse_images else 0)


def _precise_params(precise) -> jl_params:
    """Params carrying only the precision choice (for the workspace queries)."""
    return jl_params(1, 0, 1.0, 1.0, 1, 1 if precise else 0, 0)


def abi_version() -> int:
    return lib().jl_abi_version()


def group_size(L: int, w_pretrained: int) -> int:
    """[BT] §3.1: G = max(1, ceil(L / w_pretrained)) (host, exact)."""
    g = _i32()
    _check(lib().jl_group_size(int(L), int(w_pretrained), ctypes.byref(g)), "jl_group_size")
    return g.value


def rope_apply(x: torch.Tensor, positions: torch.Tensor, rope_base: float, G: int = 1,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[t, h] = R(floor(positions[t] / G)) x[t, h]; x is [T, H, d] (bf16 or fp32)."""
    _rank(x, "x", 3)
    T, H, d = x.shape
    _expect(positions.numel() == T, "positions needs T = %d entries, got %d" % (T, positions.numel()))
    _like(out, "out", tuple(x.shape), x.dtype, x.device)
    if out is None:
        out = torch.empty_like(x)
    pos = positions.to(device=x.device, dtype=torch.int32).contiguous()
    _check(lib().jl_rope_apply(_dev(out, "out"), _dev(x, "x"), _dev(pos, "positions"), T, H, d,
                               float(rope_base), int(G), _dtype(x), _stream()), "jl_rope_apply")
    return out


def prefill_workspace_bytes(T: int, n_seqs: int, Hq: int, Hkv: int, d: int, dtype,
                            precise: bool = False) -> int:
    n = ctypes.c_size_t()
    dt = JL_DTYPE_BF16 if dtype == torch.bfloat16 else JL_DTYPE_F32
    pp = _precise_params(precise)
    _check(lib().jl_bifocal_prefill_workspace(T, n_seqs, Hq, Hkv, d, dt, ctypes.byref(pp),
                                              ctypes.byref(n)),
           "jl_bifocal_prefill_workspace")
    return n.value


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    # 256-byte aligned (torch's caching allocator aligns to at least 512 bytes)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _varlen(cu_seqlens, max_seqlen, T: int, dev):
    """(cu_seqlens device tensor or None, n_seqs, max_seqlen)."""
    if cu_seqlens is None:
        return None, 1, (T if max_seqlen is None else max_seqlen)
    if isinstance(cu_seqlens, torch.Tensor):
        cu_t = cu_seqlens.to(device=dev, dtype=torch.int32).contiguous()
        if max_seqlen is None:
            max_seqlen = int((cu_t[1:] - cu_t[:-1]).max().item())
    else:
        cu_list = [int(x) for x in cu_seqlens]
        cu_t = torch.tensor(cu_list, dtype=torch.int32, device=dev)
        if max_seqlen is None:
            max_seqlen = max(b - a for a, b in zip(cu_list[:-1], cu_list[1:]))
    return cu_t, cu_t.numel() - 1, max_seqlen


def prefill_three_call_workspace_bytes(T: int, n_seqs: int, Hq: int, Hkv: int, d: int,
                                       precise: bool = False) -> int:
    n = ctypes.c_size_t()
    pp = _precise_params(precise)
    _check(lib().jl_bifocal_prefill_three_call_workspace(T, n_seqs, Hq, Hkv, d, JL_DTYPE_BF16,
                                                         ctypes.byref(pp), ctypes.byref(n)),
           "jl_bifocal_prefill_three_call_workspace")
    return n.value


def bifocal_prefill_three_call(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                               w_pretrained: int, w_local: int, rope_base: float,
                               softmax_scale: float,
                               cu_seqlens: Union[None, Sequence[int], torch.Tensor] = None,
                               max_seqlen: Optional[int] = None, precise: bool = False,
                               workspace: Optional[torch.Tensor] = None,
                               out: Optional[torch.Tensor] = None,
                               lse_out: Optional[torch.Tensor] = None
                               ) -> Tuple[torch.Tensor, torch.Tensor]:
    """The pages' unfused form ([TW] §四): three attention calls B, A, C merged in
    LogSumExp space.  bf16 only.  Returns (o [T, Hq, d], lse [Hq, T] float32)."""
    _check_qkv(q, k, v, out, lse_out)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    cu_t, n_seqs, max_seqlen = _varlen(cu_seqlens, max_seqlen, T, dev)
    o = out if out is not None else torch.empty_like(q)
    lse = lse_out if lse_out is not None else torch.empty((Hq, T), dtype=torch.float32, device=dev)
    ws = _workspace(prefill_three_call_workspace_bytes(T, n_seqs, Hq, Hkv, d, precise), dev,
                    workspace)
    p = _params(w_pretrained, w_local, rope_base, softmax_scale, True, precise)
    _check(lib().jl_bifocal_prefill_three_call(
        _dev(o, "o"), _dev(lse, "lse"), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
        None if cu_t is None else _dev(cu_t, "cu_seqlens"), n_seqs, T, int(max_seqlen), Hq, Hkv,
        d, ctypes.byref(p), _dtype(q), _dev(ws, "workspace"), ws.numel() * ws.element_size(),
        _stream()), "jl_bifocal_prefill_three_call")
    return o, lse


def bifocal_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, w_pretrained: int,
                    w_local: int, rope_base: float, softmax_scale: float, bifocal: Union[bool, int] = True,
                    cu_seqlens: Union[None, Sequence[int], torch.Tensor] = None,
                    max_seqlen: Optional[int] = None, k_rot_out: Optional[torch.Tensor] = None,
                    precise: bool = False,
                    workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    lse_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Causal bifocal prefill ([BT] §3.2): q [T, Hq, d], k/v [T, Hkv, d] raw.
    Returns (o [T, Hq, d], lse [Hq, T] float32)."""
    _check_qkv(q, k, v, out, lse_out, k_rot_out)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    cu_t, n_seqs, max_seqlen = _varlen(cu_seqlens, max_seqlen, T, dev)
    o = out if out is not None else torch.empty_like(q)
    lse = lse_out if lse_out is not None else torch.empty((Hq, T), dtype=torch.float32, device=dev)
    nbytes = prefill_workspace_bytes(T, n_seqs, Hq, Hkv, d, q.dtype, precise)
    ws = _workspace(nbytes, dev, workspace)
    p = _params(w_pretrained, w_local, rope_base, softmax_scale, bifocal, precise)
    _check(lib().jl_bifocal_prefill(
        _dev(o, "o"), _dev(lse, "lse"), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
        None if cu_t is None else _dev(cu_t, "cu_seqlens"), n_seqs, T, int(max_seqlen), Hq, Hkv,
        d, ctypes.byref(p), _dtype(q), None if k_rot_out is None else _dev(k_rot_out, "k_rot_out"),
        _dev(ws, "workspace"), ws.numel() * ws.element_size(), _stream()), "jl_bifocal_prefill")
    return o, lse


def decode_workspace_bytes(B: int, max_seqlen_k: int, Hq: int, Hkv: int, d: int, dtype) -> int:
    n = ctypes.c_size_t()
    dt = JL_DTYPE_BF16 if dtype == torch.bfloat16 else JL_DTYPE_F32
    _check(lib().jl_bifocal_decode_workspace(B, max_seqlen_k, Hq, Hkv, d, dt, ctypes.byref(n)),
           "jl_bifocal_decode_workspace")
    return n.value


def bifocal_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   seqlens_k: Union[Sequence[int], torch.Tensor], *, w_pretrained: int,
                   w_local: int, rope_base: float, softmax_scale: float, bifocal: Union[bool, int] = True,
                   max_seqlen_k: Optional[int] = None, precise: bool = False,
                   workspace: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None,
                   lse_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Bifocal decode ([TW] §三, [BT] §3.3): q [B, Hq, d] raw; caches
    [B, S_max, Hkv, d] of standard-RoPE keys.  Returns (o [B, Hq, d], lse [B, Hq])."""
    B, Hq, d = _check_cache(q, k_cache, v_cache, out, lse_out, batch_dim=True)
    _expect(k_cache.shape[0] >= B, "the caches need a row per sequence (%d), got %d"
            % (B, k_cache.shape[0]))
    _like(lse_out, "lse_out", (B, Hq), torch.float32, q.device)
    _check_lens(len(seqlens_k), B, "seqlens_k")
    S_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    if isinstance(seqlens_k, torch.Tensor):
        sl = seqlens_k.to(device=dev, dtype=torch.int32).contiguous()
        if max_seqlen_k is None:
            max_seqlen_k = int(sl.max().item())
    else:
        lens = [int(x) for x in seqlens_k]
        sl = torch.tensor(lens, dtype=torch.int32, device=dev)
        if max_seqlen_k is None:
            max_seqlen_k = max(lens)
    o = out if out is not None else torch.empty_like(q)
    lse = lse_out if lse_out is not None else torch.empty((B, Hq), dtype=torch.float32, device=dev)
    nbytes = decode_workspace_bytes(B, int(max_seqlen_k), Hq, Hkv, d, q.dtype)
    ws = _workspace(nbytes, dev, workspace)
    p = _params(w_pretrained, w_local, rope_base, softmax_scale, bifocal, precise)
    _check(lib().jl_bifocal_decode(
        _dev(o, "o"), _dev(lse, "lse"), _dev(q, "q"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(sl, "seqlens_k"), B, int(max_seqlen_k), S_max, Hq, Hkv, d,
        ctypes.byref(p), _dtype(q), _dev(ws, "workspace"), ws.numel() * ws.element_size(),
        _stream()), "jl_bifocal_decode")
    return o, lse


def bifocal_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           seqlens_k: torch.Tensor, out: torch.Tensor, lse_out: torch.Tensor, *,
                           w_pretrained: int, w_local: int, rope_base: float,
                           softmax_scale: float, max_seqlen_k: int,
                           bifocal: Union[bool, int] = True, precise: bool = False) -> None:
    """bifocal_decode on the library's static scratch (jl_bifocal_decode_noalloc):
    no workspace, and no allocation here either -- seqlens_k (int32, on the
    device), out and lse_out are the caller's.  Calls that overlap on one
    device race on that scratch."""
    B, Hq, d = _check_cache(q, k_cache, v_cache, out, lse_out, batch_dim=True)
    _expect(k_cache.shape[0] >= B, "the caches need a row per sequence")
    _like(lse_out, "lse_out", (B, Hq), torch.float32, q.device)
    _expect(seqlens_k.dtype == torch.int32 and seqlens_k.numel() == B,
            "seqlens_k must be an int32 device tensor with one entry per sequence")
    p = _params(w_pretrained, w_local, rope_base, softmax_scale, bifocal, precise)
    _check(lib().jl_bifocal_decode_noalloc(
        _dev(out, "out"), _dev(lse_out, "lse_out"), _dev(q, "q"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(seqlens_k, "seqlens_k"), B, int(max_seqlen_k),
        k_cache.shape[1], Hq, k_cache.shape[2], d, ctypes.byref(p), _dtype(q), _stream()),
        "jl_bifocal_decode_noalloc")


def decode_three_call_workspace_bytes(B: int, max_seqlen_k: int, Hq: int, Hkv: int, d: int,
                                      w_local: int) -> int:
    n = ctypes.c_size_t()
    p = jl_params(1, int(w_local), 1.0, 1.0, 1, 0)
    _check(lib().jl_bifocal_decode_three_call_workspace(B, max_seqlen_k, Hq, Hkv, d, JL_DTYPE_BF16,
                                                        ctypes.byref(p), ctypes.byref(n)),
           "jl_bifocal_decode_three_call_workspace")
    return n.value


def bifocal_decode_three_call(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              seqlens_k: Union[Sequence[int], torch.Tensor], *,
                              w_pretrained: int, w_local: int, rope_base: float,
                              softmax_scale: float, max_seqlen_k: Optional[int] = None,
                              workspace: Optional[torch.Tensor] = None,
                              out: Optional[torch.Tensor] = None,
                              lse_out: Optional[torch.Tensor] = None
                              ) -> Tuple[torch.Tensor, torch.Tensor]:
    """The pages' unfused generation step ([TW] §四): the cache's keys turned to
    remapped RoPE, three attention calls B, A, C and the LogSumExp merge.  bf16
    caches [B, S_max, Hkv, d].  Returns (o [B, Hq, d], lse [B, Hq])."""
    B, Hq, d = _check_cache(q, k_cache, v_cache, out, lse_out, batch_dim=True)
    _expect(q.dtype == torch.bfloat16, "the unfused decode takes bfloat16 tensors")
    _expect(k_cache.shape[0] >= B, "the caches need a row per sequence")
    _like(lse_out, "lse_out", (B, Hq), torch.float32, q.device)
    _check_lens(len(seqlens_k), B, "seqlens_k")
    S_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    sl, max_seqlen_k = _seqlens(seqlens_k, max_seqlen_k, dev)
    p = _params(w_pretrained, w_local, rope_base, softmax_scale, True)
    ws = _workspace(decode_three_call_workspace_bytes(B, max_seqlen_k, Hq, Hkv, d, w_local), dev,
                    workspace)
    o = out if out is not None else torch.empty_like(q)
    lse = lse_out if lse_out is not None else torch.empty((B, Hq), dtype=torch.float32, device=dev)
    _check(lib().jl_bifocal_decode_three_call(
        _dev(o, "o"), _dev(lse, "lse"), _dev(q, "q"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(sl, "seqlens_k"), B, max_seqlen_k, S_max, Hq, Hkv, d,
        ctypes.byref(p), JL_DTYPE_BF16, _dev(ws, "workspace"), ws.numel() * ws.element_size(),
        _stream()), "jl_bifocal_decode_three_call")
    return o, lse


def _seqlens(seqlens_k, max_seqlen_k, dev):
    if isinstance(seqlens_k, torch.Tensor):
        sl = seqlens_k.to(device=dev, dtype=torch.int32).contiguous()
        if max_seqlen_k is None:
            max_seqlen_k = int(sl.max().item())
    else:
        lens = [int(x) for x in seqlens_k]
        sl = torch.tensor(lens, dtype=torch.int32, device=dev)
        if max_seqlen_k is None:
            max_seqlen_k = max(lens)
    return sl, int(max_seqlen_k)


def bifocal_decode_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                         block_table: torch.Tensor, seqlens_k: Union[Sequence[int], torch.Tensor],
                         *, w_pretrained: int, w_local: int, rope_base: float,
                         softmax_scale: float, bifocal: Union[bool, int] = True,
                         max_seqlen_k: Optional[int] = None, precise: bool = False,
                         workspace: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None,
                         lse_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Bifocal decode on a paged cache: k_pages / v_pages [n_pages, page_size, Hkv, d]
    bf16, block_table [B, bt_stride] int32 (page of key j: block_table[b, j // page_size]).
    Returns (o [B, Hq, d], lse [B, Hq])."""
    B, Hq, d = _check_cache(q, k_pages, v_pages, out, lse_out, batch_dim=False)
    _like(lse_out, "lse_out", (B, Hq), torch.float32, q.device)
    _check_lens(len(seqlens_k), B, "seqlens_k")
    _check_block_table(block_table, B, block_table.device)
    n_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    dev = q.device
    sl, max_seqlen_k = _seqlens(seqlens_k, max_seqlen_k, dev)
    bt = block_table.to(device=dev, dtype=torch.int32).contiguous()
    o = out if out is not None else torch.empty_like(q)
    lse = lse_out if lse_out is not None else torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = _workspace(decode_workspace_bytes(B, max_seqlen_k, Hq, Hkv, d, q.dtype), dev, workspace)
    p = _params(w_pretrained, w_local, rope_base, softmax_scale, bifocal, precise)
    _check(lib().jl_bifocal_decode_paged(
        _dev(o, "o"), _dev(lse, "lse"), _dev(q, "q"), _dev(k_pages, "k_pages"),
        _dev(v_pages, "v_pages"), _dev(bt, "block_table"), _dev(sl, "seqlens_k"), B, max_seqlen_k,
        page_size, n_pages, bt.shape[1], Hq, Hkv, d, ctypes.byref(p), _dtype(q),
        _dev(ws, "workspace"), ws.numel() * ws.element_size(), _stream()),
        "jl_bifocal_decode_paged")
    return o, lse


def prefill_chunk_workspace_bytes(Tq: int, B: int, max_seqlen_k: int, Hq: int, Hkv: int,
                                  d: int, precise: bool = False) -> int:
    n = ctypes.c_size_t(0)
    pp = _precise_params(precise)
    _check(lib().jl_bifocal_prefill_chunk_workspace(Tq, B, max_seqlen_k, Hq, Hkv, d, 1,
                                                    ctypes.byref(pp), ctypes.byref(n)),
           "jl_bifocal_prefill_chunk_workspace")
    return n.value


def _chunk_common(q, seqlens_k, cu_seqlens_q, max_seqlen_q, max_seqlen_k, dev, out, lse_out):
    Tq, Hq, d = q.shape
    _like(lse_out, "lse_out", (Hq, Tq), torch.float32, q.device)
    cu, B, max_q = _varlen(cu_seqlens_q, max_seqlen_q, Tq, dev)
    sl, max_k = _seqlens(seqlens_k, max_seqlen_k, dev)
    if sl.numel() != B:
        raise ValueError("seqlens_k needs one entry per chunk")
    o = out if out is not None else torch.empty_like(q)
    lse = lse_out if lse_out is not None else torch.empty((Hq, Tq), dtype=torch.float32,
                                                          device=dev)
    return cu, B, max(int(max_q), 1), sl, max_k, o, lse


def bifocal_prefill_chunk(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          seqlens_k: Union[Sequence[int], torch.Tensor], *, w_pretrained: int,
                          w_local: int, rope_base: float, softmax_scale: float,
                          bifocal: Union[bool, int] = True, cu_seqlens_q=None,
                          max_seqlen_q: Optional[int] = None,
                          max_seqlen_k: Optional[int] = None, precise: bool = False,
                          reuse_images: bool = False,
                          workspace: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None,
                          lse_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunked prefill ([TW] §三, [BT] §3.1, §3.3): q [Tq, Hq, d] raw, the new
    rows of each sequence packed by cu_seqlens_q (None: one chunk); caches
    [B, S_max, Hkv, d] bf16 of standard-RoPE keys holding seqlens_k[b] keys,
    the chunk's own included.  reuse_images (with a workspace the caller
    keeps across the chunks of a prefill, sized for the largest chunk, and
    the same max_seqlen_k every call): cache rows already turned by an
    earlier call are not turned again.  The first chunk of a prefill passes
    False (the workspace may hold images of other caches).
    Returns (o [Tq, Hq, d], lse [Hq, Tq])."""
    _expect(workspace is not None or not reuse_images,
            "reuse_images needs a workspace the caller keeps between calls")
    _check_cache(q, k_cache, v_cache, out, None, batch_dim=True)
    _expect(q.dtype == torch.bfloat16, "chunked prefill takes bfloat16 tensors")
    _check_lens(len(seqlens_k), 1 if cu_seqlens_q is None else len(cu_seqlens_q) - 1, "seqlens_k")
    _expect(k_cache.shape[0] >= len(seqlens_k), "the caches need a row per sequence")
    dev = q.device
    Hq, d = q.shape[1], q.shape[2]
    S_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    cu, B, max_q, sl, max_k, o, lse = _chunk_common(q, seqlens_k, cu_seqlens_q, max_seqlen_q,
                                                    max_seqlen_k, dev, out, lse_out)
    ws = _workspace(prefill_chunk_workspace_bytes(q.shape[0], B, max_k, Hq, Hkv, d, precise), dev,
                    workspace)
    p = _params(w_pretrained, w_local, rope_base, softmax_scale, bifocal, precise, reuse_images)
    _check(lib().jl_bifocal_prefill_chunk(
        _dev(o, "o"), _dev(lse, "lse"), _dev(q, "q"), None if cu is None else _dev(cu, "cu"),
        q.shape[0], max_q, _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(sl, "seqlens_k"), B, max_k, S_max, Hq, Hkv, d, ctypes.byref(p), _dtype(q),
        _dev(ws, "workspace"), ws.numel() * ws.element_size(), _stream()),
        "jl_bifocal_prefill_chunk")
    return o, lse


def bifocal_prefill_chunk_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                                block_table: torch.Tensor,
                                seqlens_k: Union[Sequence[int], torch.Tensor], *,
                                w_pretrained: int, w_local: int, rope_base: float,
                                softmax_scale: float, bifocal: Union[bool, int] = True, cu_seqlens_q=None,
                                max_seqlen_q: Optional[int] = None,
                                max_seqlen_k: Optional[int] = None, precise: bool = False,
                                reuse_images: bool = False,
                                workspace: Optional[torch.Tensor] = None,
                                out: Optional[torch.Tensor] = None,
                                lse_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """bifocal_prefill_chunk on a paged cache: k_pages / v_pages
    [n_pages, page_size, Hkv, d] bf16, block_table [B, bt_stride] int32."""
    _expect(workspace is not None or not reuse_images,
            "reuse_images needs a workspace the caller keeps between calls")
    _check_cache(q, k_pages, v_pages, out, None, batch_dim=False)
    _expect(q.dtype == torch.bfloat16, "chunked prefill takes bfloat16 tensors")
    nb = 1 if cu_seqlens_q is None else len(cu_seqlens_q) - 1
    _check_lens(len(seqlens_k), nb, "seqlens_k")
    _check_block_table(block_table, nb, block_table.device)
    dev = q.device
    Hq, d = q.shape[1], q.shape[2]
    n_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    cu, B, max_q, sl, max_k, o, lse = _chunk_common(q, seqlens_k, cu_seqlens_q, max_seqlen_q,
                                                    max_seqlen_k, dev, out, lse_out)
    bt = block_table.to(device=dev, dtype=torch.int32).contiguous()
    ws = _workspace(prefill_chunk_workspace_bytes(q.shape[0], B, max_k, Hq, Hkv, d, precise), dev,
                    workspace)
    p = _params(w_pretrained, w_local, rope_base, softmax_scale, bifocal, precise, reuse_images)
    _check(lib().jl_bifocal_prefill_chunk_paged(
        _dev(o, "o"), _dev(lse, "lse"), _dev(q, "q"), None if cu is None else _dev(cu, "cu"),
        q.shape[0], max_q, _dev(k_pages, "k_pages"), _dev(v_pages, "v_pages"),
        _dev(bt, "block_table"), _dev(sl, "seqlens_k"), B, max_k, page_size, n_pages,
        bt.shape[1], Hq, Hkv, d, ctypes.byref(p), _dtype(q), _dev(ws, "workspace"),
        ws.numel() * ws.element_size(), _stream()),
        "jl_bifocal_prefill_chunk_paged")
    return o, lse


def _u8(t: torch.Tensor, name: str) -> int:
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise ValueError("%s must hold E4M3 codes (uint8 or float8_e4m3fn)" % name)
    return _dev(t, name)


def _scale(x, H: int, dev) -> torch.Tensor:
    if isinstance(x, torch.Tensor):
        return x.to(device=dev, dtype=torch.float32).contiguous().reshape(H)
    return torch.tensor([float(v) for v in x], dtype=torch.float32, device=dev).reshape(H)


def kv_quantize_fp8(x: torch.Tensor, scale, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """E4M3 codes (uint8) of x / scale[h] for a bf16 cache block x [..., H, d]."""
    _expect(x.dim() >= 2 and x.dtype == torch.bfloat16, "x must be a bfloat16 [..., H, d] tensor")
    if out is not None:
        _expect(tuple(out.shape) == tuple(x.shape) and out.device == x.device,
                "out must have x's shape %s and device" % (tuple(x.shape),))
    H, d = x.shape[-2], x.shape[-1]
    sc = _scale(scale, H, x.device)
    o = out if out is not None else torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(lib().jl_kv_quantize_fp8(_u8(o, "out"), _dev(x, "x"), _dev(sc, "scale"),
                                    x.numel() // (H * d), H, d, _stream()),
           "jl_kv_quantize_fp8")
    return o


def bifocal_decode_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale,
                       v_scale, seqlens_k: Union[Sequence[int], torch.Tensor], *,
                       w_pretrained: int, w_local: int, rope_base: float, softmax_scale: float,
                       bifocal: Union[bool, int] = True, max_seqlen_k: Optional[int] = None,
                       block_table: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None,
                       lse_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Bifocal decode on an fp8 (E4M3) cache with per-kv-head scales.  Flat
    caches [B, S_max, Hkv, d]; with ``block_table`` page pools
    [n_pages, page_size, Hkv, d].  Returns (o [B, Hq, d], lse [B, Hq])."""
    B, Hq, d = _check_cache(q, k_cache, v_cache, out, lse_out, batch_dim=block_table is None,
                            cache_dtype=(torch.uint8, torch.float8_e4m3fn))
    _expect(q.dtype == torch.bfloat16, "fp8 decode takes bfloat16 queries")
    _like(lse_out, "lse_out", (B, Hq), torch.float32, q.device)
    _check_lens(len(seqlens_k), B, "seqlens_k")
    if block_table is None:
        _expect(k_cache.shape[0] >= B, "the caches need a row per sequence (%d), got %d"
                % (B, k_cache.shape[0]))
    else:
        _check_block_table(block_table, B, block_table.device)
    dev = q.device
    Hkv = k_cache.shape[2]
    sl, max_seqlen_k = _seqlens(seqlens_k, max_seqlen_k, dev)
    ks, vs = _scale(k_scale, Hkv, dev), _scale(v_scale, Hkv, dev)
    o = out if out is not None else torch.empty_like(q)
    lse = lse_out if lse_out is not None else torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = _workspace(decode_workspace_bytes(B, max_seqlen_k, Hq, Hkv, d, torch.bfloat16), dev,
                    workspace)
    p = _params(w_pretrained, w_local, rope_base, softmax_scale, bifocal)
    if block_table is None:
        _check(lib().jl_bifocal_decode_fp8(
            _dev(o, "o"), _dev(lse, "lse"), _dev(q, "q"), _u8(k_cache, "k_cache"),
            _u8(v_cache, "v_cache"), _dev(ks, "k_scale"), _dev(vs, "v_scale"),
            _dev(sl, "seqlens_k"), B, max_seqlen_k, k_cache.shape[1], Hq, Hkv, d,
            ctypes.byref(p), _dev(ws, "workspace"), ws.numel() * ws.element_size(), _stream()),
            "jl_bifocal_decode_fp8")
    else:
        bt = block_table.to(device=dev, dtype=torch.int32).contiguous()
        _check(lib().jl_bifocal_decode_fp8_paged(
            _dev(o, "o"), _dev(lse, "lse"), _dev(q, "q"), _u8(k_cache, "k_pages"),
            _u8(v_cache, "v_pages"), _dev(ks, "k_scale"), _dev(vs, "v_scale"),
            _dev(bt, "block_table"), _dev(sl, "seqlens_k"), B, max_seqlen_k, k_cache.shape[1],
            k_cache.shape[0], bt.shape[1], Hq, Hkv, d, ctypes.byref(p), _dev(ws, "workspace"),
            ws.numel() * ws.element_size(), _stream()),
            "jl_bifocal_decode_fp8_paged")
    return o, lse


def debug_index_math(L: int, w_pretrained: int, w_local: int, bifocal: bool, bm: int, bn: int,
                     device="cuda"):
    """Runs the kernels' device index functions; returns (G, f, band, tile) on the host."""
    n = min(L, 1024)
    nti, ntj = (L + bm - 1) // bm, (L + bn - 1) // bn
    G = torch.zeros(1, dtype=torch.int32, device=device)
    f = torch.zeros(L, dtype=torch.int32, device=device)
    band = torch.zeros(n * n, dtype=torch.uint8, device=device)
    tile = torch.zeros(nti * ntj, dtype=torch.uint8, device=device)
    _check(lib().jl_debug_index_math(int(L), int(w_pretrained), int(w_local), 1 if bifocal else 0,
                                     int(bm), int(bn), G.data_ptr(), f.data_ptr(), band.data_ptr(),
                                     tile.data_ptr(), _stream()), "jl_debug_index_math")
    torch.cuda.synchronize(device)
    return (int(G.item()), f.cpu().numpy(), band.cpu().numpy().reshape(n, n),
            tile.cpu().numpy().reshape(nti, ntj))


def stream_read(buf: torch.Tensor, partial: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Reads every byte of the contiguous device tensor `buf` once
    (jl_debug_stream_read); returns the 256 per-workgroup wrapping uint32 sums
    (as int32, on the device, not synchronized)."""
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    nbytes = buf.numel() * buf.element_size()
    if partial is None:
        partial = torch.empty(256, dtype=torch.int32, device=buf.device)
    _check(lib().jl_debug_stream_read(buf.data_ptr(), nbytes, partial.data_ptr(), _stream()),
           "jl_debug_stream_read")
    return partial


MFMA_STREAM_OPERAND_BYTES = 256 * 512 * 16 * 16


def mfma_stream(operands: torch.Tensor, iters: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Runs the matrix-core stream (jl_debug_mfma_stream) on the contiguous
    fp16 device tensor `operands` (at least MFMA_STREAM_OPERAND_BYTES bytes);
    returns the 131072 per-thread accumulator sums (fp32, on the device, not
    synchronized).  One call performs 256 * 8 * iters * 32 MFMAs of 32768 flops."""
    if operands.dtype != torch.float16 or not operands.is_contiguous():
        raise ValueError("operands must be a contiguous float16 tensor")
    nbytes = operands.numel() * operands.element_size()
    if out is None:
        out = torch.empty(256 * 512, dtype=torch.float32, device=operands.device)
    if out.dtype != torch.float32 or out.numel() < 256 * 512 or out.device != operands.device:
        raise ValueError("out must be a float32 tensor of at least 131072 elements on the operands' device")
    _check(lib().jl_debug_mfma_stream(operands.data_ptr(), nbytes, int(iters), out.data_ptr(), _stream()),
           "jl_debug_mfma_stream")
    return out


def profile_enable(on: bool) -> None:
    _check(lib().jl_profile_enable(1 if on else 0), "jl_profile_enable")


def profile_read() -> dict:
    """{kernel name: (launch count, total ms)} since the last enable/read."""
    cap = 64
    names = (ctypes.c_char_p * cap)()
    counts = (_i32 * cap)()
    tot = (ctypes.c_double * cap)()
    n = _i32()
    _check(lib().jl_profile_read(names, counts, tot, cap, ctypes.byref(n)), "jl_profile_read")
    return {names[i].decode(): (counts[i], tot[i]) for i in range(min(n.value, cap))}

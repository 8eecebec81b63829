"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call
(fake, never-dereferenced pointers are enough to reach each check)."""
import ctypes
import os
import re

import pytest

from long_context_attention_jl_amd import jetlong as jlb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "jetlong.h")

FAKE = 0x100000  # 256-byte aligned, never dereferenced by a failing call


def _declared():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(jl_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for must in ("jl_rope_apply", "jl_bifocal_prefill", "jl_bifocal_decode", "jl_group_size",
                 "jl_bifocal_prefill_workspace", "jl_bifocal_decode_workspace"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(jlb.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_abi_version_and_status_strings():
    assert jlb.abi_version() == 3
    L = jlb.lib()
    assert L.jl_status_string(0) == b"JL_OK"
    assert L.jl_status_string(4) == b"JL_ERR_HIP"
    assert L.jl_status_string(99) == b"JL_UNKNOWN_STATUS"


@pytest.mark.parametrize("L,w,G", [(65536, 32768, 2), (131072, 32768, 4), (32768, 32768, 1),
                                   (32769, 32768, 2), (1, 1, 1), (512, 128, 4), (98304, 32768, 3)])
def test_group_size_host(L, w, G):
    assert jlb.group_size(L, w) == G


def test_group_size_rejects():
    with pytest.raises(jlb.JLError) as e:
        jlb.group_size(0, 5)
    assert e.value.status == jlb.JL_ERR_INVALID_ARGUMENT
    with pytest.raises(jlb.JLError):
        jlb.group_size(5, 0)


def _params(**kw):
    d = dict(w_pretrained=32768, w_local=2048, rope_base=1e6, softmax_scale=0.088, bifocal=1,
             precise=0, reuse_images=0)
    d.update(kw)
    return jlb.jl_params(d["w_pretrained"], d["w_local"], d["rope_base"], d["softmax_scale"],
                         d["bifocal"], d["precise"], d["reuse_images"])


def _prefill(**kw):
    a = dict(o=FAKE, lse=FAKE * 2, q=FAKE * 3, k=FAKE * 4, v=FAKE * 5, cu=None, n_seqs=1, T=1024,
             max_seqlen=1024, Hq=32, Hkv=8, d=128, params=_params(), dtype=1, krot=None,
             ws=FAKE * 8, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    p = a["params"]
    return jlb.lib().jl_bifocal_prefill(
        a["o"], a["lse"], a["q"], a["k"], a["v"], a["cu"], a["n_seqs"], a["T"], a["max_seqlen"],
        a["Hq"], a["Hkv"], a["d"], None if p is None else ctypes.byref(p), a["dtype"], a["krot"],
        a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), 1), (dict(q=None), 1), (dict(ws=None), 1), (dict(params=None), 1),
    (dict(T=0), 1), (dict(n_seqs=0), 1), (dict(n_seqs=2), 1), (dict(max_seqlen=0), 1),
    (dict(max_seqlen=2000), 1), (dict(max_seqlen=512), 1), (dict(Hq=30), 1), (dict(Hkv=0), 1),
    (dict(d=96), 2), (dict(d=65), 1), (dict(dtype=7), 2),
    (dict(params=_params(w_pretrained=0)), 1), (dict(params=_params(w_local=-1)), 1),
    (dict(params=_params(rope_base=0.0)), 1), (dict(params=_params(softmax_scale=0.0)), 1),
    (dict(params=_params(softmax_scale=float("inf"))), 1), (dict(params=_params(bifocal=3)), 1),
    (dict(params=_params(bifocal=-1)), 1), (dict(params=_params(bifocal=2), dtype=0), 2),
    (dict(params=_params(precise=2)), 1), (dict(params=_params(precise=-1)), 1),
    (dict(params=_params(reuse_images=2)), 1),
    (dict(ws_bytes=1000), 3), (dict(ws=FAKE * 8 + 4), 1), (dict(o=FAKE * 3), 1),
    (dict(krot=FAKE * 4), 1), (dict(cu=FAKE * 9, n_seqs=70000, T=1 << 20, max_seqlen=1024), 2),
])
def test_prefill_validation(kw, status):
    assert _prefill(**kw) == status
    assert jlb.lib().jl_last_error()


def _three_call(**kw):
    a = dict(o=FAKE, lse=FAKE * 2, q=FAKE * 3, k=FAKE * 4, v=FAKE * 5, cu=None, n_seqs=1, T=1024,
             max_seqlen=1024, Hq=32, Hkv=8, d=128, params=_params(), dtype=1,
             ws=FAKE * 8, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    p = a["params"]
    return jlb.lib().jl_bifocal_prefill_three_call(
        a["o"], a["lse"], a["q"], a["k"], a["v"], a["cu"], a["n_seqs"], a["T"], a["max_seqlen"],
        a["Hq"], a["Hkv"], a["d"], None if p is None else ctypes.byref(p), a["dtype"],
        a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), 1), (dict(ws=None), 1), (dict(params=None), 1), (dict(T=0), 1),
    (dict(n_seqs=2), 1), (dict(max_seqlen=2000), 1), (dict(Hq=30), 1), (dict(d=96), 2),
    (dict(dtype=0), 2), (dict(params=_params(bifocal=0)), 1), (dict(params=_params(bifocal=2)), 1),
    (dict(ws_bytes=1000), 3),
    (dict(ws=FAKE * 8 + 4), 1), (dict(o=FAKE * 3), 1),
])
def test_three_call_validation(kw, status):
    assert _three_call(**kw) == status
    assert jlb.lib().jl_last_error()


def test_three_call_workspace_query():
    n = ctypes.c_size_t()
    m = ctypes.c_size_t()
    L = jlb.lib()
    assert L.jl_bifocal_prefill_three_call_workspace(4096, 1, 32, 8, 128, 1, None, ctypes.byref(n)) == 0
    assert L.jl_bifocal_prefill_workspace(4096, 1, 32, 8, 128, 1, None, ctypes.byref(m)) == 0
    # the three calls' bf16 outputs and fp32 LSEs come on top of the prefill workspace
    assert n.value >= m.value + 3 * (4096 * 32 * 128 * 2 + 32 * 4096 * 4)
    assert L.jl_bifocal_prefill_three_call_workspace(4096, 1, 32, 8, 128, 0, None, ctypes.byref(n)) == 2


def test_prefill_workspace_query():
    n = ctypes.c_size_t()
    L = jlb.lib()
    assert L.jl_bifocal_prefill_workspace(131072, 1, 32, 8, 128, 1, None, ctypes.byref(n)) == 0
    # three bf16 key/value layouts of the padded sequence dominate
    assert n.value >= 3 * 8 * 131072 * 128 * 2
    assert L.jl_bifocal_prefill_workspace(512, 1, 1, 1, 64, 0, None, ctypes.byref(n)) == 0
    assert n.value >= 2 * 512 * 64 * 4
    assert L.jl_bifocal_prefill_workspace(0, 1, 1, 1, 64, 0, None, ctypes.byref(n)) == 1
    assert L.jl_bifocal_prefill_workspace(10, 1, 3, 2, 64, 0, None, ctypes.byref(n)) == 1
    assert L.jl_bifocal_prefill_workspace(10, 1, 1, 1, 80, 0, None, ctypes.byref(n)) == 2


def _decode(**kw):
    a = dict(o=FAKE, lse=FAKE * 2, q=FAKE * 3, kc=FAKE * 4, vc=FAKE * 5, sl=FAKE * 6, B=1,
             max_L=131072, S_max=131072, Hq=32, Hkv=8, d=128, params=_params(), dtype=1,
             ws=FAKE * 8, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    p = a["params"]
    return jlb.lib().jl_bifocal_decode(
        a["o"], a["lse"], a["q"], a["kc"], a["vc"], a["sl"], a["B"], a["max_L"], a["S_max"],
        a["Hq"], a["Hkv"], a["d"], None if p is None else ctypes.byref(p), a["dtype"], a["ws"],
        a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), 1), (dict(sl=None), 1), (dict(kc=None), 1), (dict(B=0), 1),
    (dict(max_L=0), 1), (dict(S_max=100), 1), (dict(Hq=33), 1), (dict(Hq=34, Hkv=2), 2),
    (dict(d=32), 2), (dict(dtype=3), 2), (dict(params=_params(w_local=-5)), 1),
    (dict(ws_bytes=16), 3), (dict(ws=FAKE * 8 + 128), 1), (dict(o=FAKE * 4), 1),
    (dict(B=70000), 2), (dict(params=_params(bifocal=2), dtype=0), 2),
    (dict(params=_params(bifocal=5)), 1),
])
def test_decode_validation(kw, status):
    assert _decode(**kw) == status


def test_rope_validation():
    L = jlb.lib()
    assert L.jl_rope_apply(None, FAKE, FAKE, 10, 1, 64, 1e4, 1, 1, None) == 1
    assert L.jl_rope_apply(FAKE, FAKE, FAKE, 0, 1, 64, 1e4, 1, 1, None) == 1
    assert L.jl_rope_apply(FAKE, FAKE, FAKE, 10, 1, 48, 1e4, 1, 1, None) == 2
    assert L.jl_rope_apply(FAKE, FAKE, FAKE, 10, 1, 64, -1.0, 1, 1, None) == 1
    assert L.jl_rope_apply(FAKE, FAKE, FAKE, 10, 1, 64, 1e4, 0, 1, None) == 1


def test_debug_and_profile_validation():
    L = jlb.lib()
    assert L.jl_debug_index_math(0, 8, 2, 1, 16, 16, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.jl_debug_index_math(10, 8, 2, 1, 0, 16, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.jl_debug_index_math(10, 8, 2, 1, 16, 16, None, FAKE, FAKE, FAKE, None) == 1
    n = ctypes.c_int32()
    assert L.jl_profile_read(None, None, None, 0, ctypes.byref(n)) == 0
    assert n.value == 0
    assert L.jl_profile_read(None, None, None, 0, None) == 1


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(jlb, "_lib", None)
    monkeypatch.setattr(jlb, "LIB_PATH", "/nonexistent/libjetlong.so")
    with pytest.raises(RuntimeError):
        jlb.lib()


def _paged(**kw):
    a = dict(o=FAKE, lse=FAKE * 2, q=FAKE * 3, kp=FAKE * 4, vp=FAKE * 5, bt=FAKE * 6, sl=FAKE * 7,
             B=2, max_len=4096, page=64, n_pages=200, bt_stride=64, Hq=32, Hkv=8, d=128,
             params=_params(), dtype=1, ws=FAKE * 8, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    p = a["params"]
    return jlb.lib().jl_bifocal_decode_paged(
        a["o"], a["lse"], a["q"], a["kp"], a["vp"], a["bt"], a["sl"], a["B"], a["max_len"],
        a["page"], a["n_pages"], a["bt_stride"], a["Hq"], a["Hkv"], a["d"],
        None if p is None else ctypes.byref(p), a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(bt=None), 1), (dict(kp=None), 1), (dict(B=0), 1), (dict(page=48), 1), (dict(page=8), 1),
    (dict(n_pages=0), 1), (dict(bt_stride=63), 1), (dict(Hq=30), 1), (dict(Hq=32, Hkv=1), 2),
    (dict(dtype=0), 2), (dict(d=96), 2), (dict(ws_bytes=100), 3), (dict(ws=FAKE * 8 + 4), 1),
    (dict(o=FAKE * 3), 1), (dict(params=_params(w_pretrained=0)), 1),
])
def test_paged_decode_validation(kw, status):
    assert _paged(**kw) == status
    assert jlb.lib().jl_last_error()


def _chunk(paged=False, **kw):
    a = dict(o=FAKE, lse=FAKE * 2, q=FAKE * 3, cu=FAKE * 4, Tq=512, max_q=512, kc=FAKE * 5,
             vc=FAKE * 6, bt=FAKE * 9, sl=FAKE * 7, B=2, max_k=4096, S_max=4096, page=64,
             n_pages=200, bt_stride=64, Hq=32, Hkv=8, d=128, params=_params(), dtype=1,
             ws=FAKE * 8, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    p = a["params"]
    pp = None if p is None else ctypes.byref(p)
    L = jlb.lib()
    if paged:
        return L.jl_bifocal_prefill_chunk_paged(
            a["o"], a["lse"], a["q"], a["cu"], a["Tq"], a["max_q"], a["kc"], a["vc"], a["bt"],
            a["sl"], a["B"], a["max_k"], a["page"], a["n_pages"], a["bt_stride"], a["Hq"],
            a["Hkv"], a["d"], pp, a["dtype"], a["ws"], a["ws_bytes"], a["stream"])
    return L.jl_bifocal_prefill_chunk(
        a["o"], a["lse"], a["q"], a["cu"], a["Tq"], a["max_q"], a["kc"], a["vc"], a["sl"], a["B"],
        a["max_k"], a["S_max"], a["Hq"], a["Hkv"], a["d"], pp, a["dtype"], a["ws"],
        a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(sl=None), 1), (dict(kc=None), 1), (dict(params=None), 1),
    (dict(B=0), 1), (dict(B=70000), 2), (dict(Tq=0), 1), (dict(max_q=0), 1),
    (dict(max_q=513), 1), (dict(max_q=5000, Tq=6000), 1), (dict(cu=None), 1),
    (dict(cu=None, B=1, max_q=100), 1), (dict(max_k=0), 1), (dict(B=600, max_k=4000000, S_max=4000000, bt_stride=70000), 2),
    (dict(Hq=30), 1), (dict(Hq=32, Hkv=64), 1), (dict(dtype=0), 2), (dict(d=96), 2),
    (dict(o=FAKE * 3), 1), (dict(ws=FAKE * 8 + 4), 1), (dict(ws_bytes=100), 3),
    (dict(params=_params(w_pretrained=0)), 1),
])
def test_chunk_validation(paged, kw, status):
    assert _chunk(paged, **kw) == status
    assert jlb.lib().jl_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(S_max=4095), 1), (dict(S_max=0, max_k=1), 1),
])
def test_chunk_flat_validation(kw, status):
    assert _chunk(False, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(bt=None), 1), (dict(page=48), 1), (dict(page=8), 1), (dict(n_pages=0), 1),
    (dict(bt_stride=63), 1), (dict(n_pages=1 << 40), 1),
])
def test_chunk_paged_validation(kw, status):
    assert _chunk(True, **kw) == status


def test_chunk_workspace_query():
    """A large chunk needs the prefill workspace of its keys plus the 256-byte
    record of the images; a grid of fewer workgroups than compute units (256)
    adds the key-split partials: up to 4 shares x Tq x Hq x (d + 2) fp32."""
    n = ctypes.c_size_t(0)
    L = jlb.lib()
    assert L.jl_bifocal_prefill_workspace(131072, 1, 32, 8, 128, 1, None, ctypes.byref(n)) == 0
    base = n.value + 256
    # 32768 rows of 32 heads: 4096 row blocks >= 1024 workgroups, no split
    assert L.jl_bifocal_prefill_chunk_workspace(32768, 1, 131072, 32, 8, 128, 1, None, ctypes.byref(n)) == 0
    assert n.value == base
    # 4096 and 2048 rows: 512 and 256 row-block workgroups, at least one per
    # compute unit: no split
    assert L.jl_bifocal_prefill_chunk_workspace(4096, 1, 131072, 32, 8, 128, 1, None, ctypes.byref(n)) == 0
    assert n.value == base
    assert L.jl_bifocal_prefill_chunk_workspace(2048, 1, 131072, 32, 8, 128, 1, None, ctypes.byref(n)) == 0
    assert n.value == base
    # 1024 rows: 128 workgroups -> 2 shares
    assert L.jl_bifocal_prefill_chunk_workspace(1024, 1, 131072, 32, 8, 128, 1, None, ctypes.byref(n)) == 0
    assert base + 2 * 1024 * 32 * 130 * 4 <= n.value < base + 2 * 1024 * 32 * 130 * 4 + 1024
    # 512 rows: 64 workgroups -> 4 shares
    assert L.jl_bifocal_prefill_chunk_workspace(512, 1, 131072, 32, 8, 128, 1, None, ctypes.byref(n)) == 0
    assert base + 4 * 512 * 32 * 130 * 4 <= n.value < base + 4 * 512 * 32 * 130 * 4 + 1024
    # one row: capped at 4 shares
    assert L.jl_bifocal_prefill_chunk_workspace(1, 1, 131072, 32, 8, 128, 1, None, ctypes.byref(n)) == 0
    assert base + 4 * 32 * 130 * 4 <= n.value < base + 4 * 32 * 130 * 4 + 1024
    assert L.jl_bifocal_prefill_chunk_workspace(1, 1, 131072, 32, 8, 128, 0, None, ctypes.byref(n)) == 2
    assert L.jl_bifocal_prefill_chunk_workspace(1, 0, 10, 32, 8, 128, 1, None, ctypes.byref(n)) == 1
    assert L.jl_bifocal_prefill_chunk_workspace(0, 1, 10, 32, 8, 128, 1, None, ctypes.byref(n)) == 1
    assert L.jl_bifocal_prefill_chunk_workspace(1, 1, 10, 32, 8, 128, 1, None, None) == 1


def _fp8(paged=False, **kw):
    a = dict(o=FAKE, lse=FAKE * 2, q=FAKE * 3, kc=FAKE * 4, vc=FAKE * 5, ks=FAKE * 9,
             vs=FAKE * 10, bt=FAKE * 6, sl=FAKE * 7, B=2, max_len=4096, S_max=4096, page=64,
             n_pages=200, bt_stride=64, Hq=32, Hkv=8, d=128, params=_params(), ws=FAKE * 8,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    p = a["params"]
    pp = None if p is None else ctypes.byref(p)
    L = jlb.lib()
    if paged:
        return L.jl_bifocal_decode_fp8_paged(
            a["o"], a["lse"], a["q"], a["kc"], a["vc"], a["ks"], a["vs"], a["bt"], a["sl"],
            a["B"], a["max_len"], a["page"], a["n_pages"], a["bt_stride"], a["Hq"], a["Hkv"],
            a["d"], pp, a["ws"], a["ws_bytes"], a["stream"])
    return L.jl_bifocal_decode_fp8(
        a["o"], a["lse"], a["q"], a["kc"], a["vc"], a["ks"], a["vs"], a["sl"], a["B"],
        a["max_len"], a["S_max"], a["Hq"], a["Hkv"], a["d"], pp, a["ws"], a["ws_bytes"],
        a["stream"])


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(ks=None), 1), (dict(vs=None), 1), (dict(kc=None), 1), (dict(sl=None), 1),
    (dict(params=None), 1), (dict(B=0), 1), (dict(B=70000), 2), (dict(max_len=0), 1),
    (dict(Hq=30), 1), (dict(Hq=32, Hkv=1), 2), (dict(d=96), 2), (dict(ws_bytes=100), 3),
    (dict(ws=FAKE * 8 + 4), 1), (dict(o=FAKE * 3), 1),
])
def test_fp8_decode_validation(paged, kw, status):
    assert _fp8(paged, **kw) == status
    assert jlb.lib().jl_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(bt=None), 1), (dict(page=48), 1), (dict(n_pages=0), 1), (dict(bt_stride=63), 1),
])
def test_fp8_paged_decode_validation(kw, status):
    assert _fp8(True, **kw) == status


def test_fp8_decode_workspace_is_the_bf16_one():
    """The fp8 decode call accepts exactly the bf16 decode workspace size."""
    n = ctypes.c_size_t(0)
    assert jlb.lib().jl_bifocal_decode_workspace(2, 4096, 32, 8, 128, 1, ctypes.byref(n)) == 0
    assert _fp8(ws_bytes=n.value - 1) == 3


@pytest.mark.parametrize("args,status", [
    ((None, FAKE, FAKE * 2, 10, 8, 128), 1), ((FAKE, None, FAKE * 2, 10, 8, 128), 1),
    ((FAKE, FAKE * 3, None, 10, 8, 128), 1), ((FAKE, FAKE * 3, FAKE * 2, 0, 8, 128), 1),
    ((FAKE, FAKE * 3, FAKE * 2, 10, 0, 128), 1), ((FAKE, FAKE * 3, FAKE * 2, 10, 8, 100), 1),
    ((FAKE + 4, FAKE * 3, FAKE * 2, 10, 8, 128), 1), ((FAKE, FAKE * 3 + 8, FAKE * 2, 10, 8, 128), 1),
    ((FAKE, FAKE, FAKE * 2, 10, 8, 128), 1),
])
def test_kv_quantize_validation(args, status):
    assert jlb.lib().jl_kv_quantize_fp8(*args, None) == status


@pytest.mark.parametrize("call,kw", [
    (_prefill, dict(q=FAKE * 3 + 8)), (_prefill, dict(o=FAKE + 2)),
    (_prefill, dict(krot=FAKE * 9 + 4)), (_three_call, dict(v=FAKE * 5 + 8)),
    (_decode, dict(kc=FAKE * 4 + 8)), (_decode, dict(q=FAKE * 3 + 2)),
    (_paged, dict(vp=FAKE * 5 + 4)), (_chunk, dict(o=FAKE + 8)),
    (lambda **kw: _chunk(True, **kw), dict(kc=FAKE * 5 + 8)), (_fp8, dict(vc=FAKE * 5 + 8)),
])
def test_vector_operands_must_be_16_byte_aligned(call, kw):
    """Every attention kernel moves q, k, v, o and the caches in 16-byte
    vectors; a pointer off that boundary is refused on the host."""
    assert call(**kw) == 1
    assert b"16-byte" in jlb.lib().jl_last_error()


@pytest.mark.parametrize("args,status", [
    ((None, 1024, FAKE), 1), ((FAKE, 1024, None), 1), ((FAKE, 0, FAKE), 1), ((FAKE, 24, FAKE), 1),
    ((FAKE + 8, 1024, FAKE), 1), ((FAKE, 1024, FAKE + 2), 1),
])
def test_stream_read_validation(args, status):
    assert jlb.lib().jl_debug_stream_read(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((None, 1 << 25, 1, FAKE), 1), ((FAKE, 1 << 25, 1, None), 1), ((FAKE, (1 << 25) - 16, 1, FAKE), 1),
    ((FAKE, 1 << 25, 0, FAKE), 1), ((FAKE, 1 << 25, (1 << 24) + 1, FAKE), 1),
    ((FAKE + 8, 1 << 25, 1, FAKE), 1), ((FAKE, 1 << 25, 1, FAKE + 2), 1),
])
def test_mfma_stream_validation(args, status):
    assert jlb.lib().jl_debug_mfma_stream(*args, None) == status


# ---- the Python binding checks every tensor against q before any call --------
# (CPU tensors: the shape/dtype checks run before the device check, so no
# pointer reaches the library.)

def _t(*shape, dtype=None):
    import torch
    return torch.zeros(*shape, dtype=dtype or torch.bfloat16)


_PF = dict(w_pretrained=64, w_local=8, rope_base=1e4, softmax_scale=0.1)


@pytest.mark.parametrize("case", [
    "k_dtype", "v_shape", "k_head_dim", "k_tokens", "out_dtype", "out_shape", "lse_dtype",
    "lse_shape", "k_rot_shape", "k_rot_dtype",
])
def test_binding_prefill_rejects_mismatched_tensors(case):
    import torch
    q, k, v = _t(100, 4, 64), _t(100, 2, 64), _t(100, 2, 64)
    extra = {}
    if case == "k_dtype":
        k = _t(100, 2, 64, dtype=torch.float32)
    elif case == "v_shape":
        v = _t(100, 1, 64)
    elif case == "k_head_dim":
        k = _t(100, 2, 128)
    elif case == "k_tokens":
        k = _t(99, 2, 64)
    elif case == "out_dtype":
        extra["out"] = _t(100, 4, 64, dtype=torch.float32)
    elif case == "out_shape":
        extra["out"] = _t(100, 4, 32)
    elif case == "lse_dtype":
        extra["lse_out"] = _t(4, 100)
    elif case == "lse_shape":
        extra["lse_out"] = _t(100, 4, dtype=torch.float32)
    elif case == "k_rot_shape":
        extra["k_rot_out"] = _t(100, 4, 64)
    elif case == "k_rot_dtype":
        extra["k_rot_out"] = _t(100, 2, 64, dtype=torch.float32)
    with pytest.raises(ValueError):
        jlb.bifocal_prefill(q, k, v, **_PF, **extra)
    if case != "k_rot_shape" and case != "k_rot_dtype":
        with pytest.raises(ValueError):
            jlb.bifocal_prefill_three_call(q, k, v, **_PF, **extra)


@pytest.mark.parametrize("case", [
    "cache_batch", "cache_dtype", "cache_head_dim", "v_shape", "out_dtype", "lse_shape",
    "seqlens_count", "heads",
])
def test_binding_decode_rejects_mismatched_tensors(case):
    import torch
    q, kc, vc = _t(2, 4, 64), _t(2, 50, 2, 64), _t(2, 50, 2, 64)
    lens, extra = [50, 10], {}
    if case == "cache_batch":
        kc, vc = _t(1, 50, 2, 64), _t(1, 50, 2, 64)
    elif case == "cache_dtype":
        kc = _t(2, 50, 2, 64, dtype=torch.float32)
    elif case == "cache_head_dim":
        kc, vc = _t(2, 50, 2, 128), _t(2, 50, 2, 128)
    elif case == "v_shape":
        vc = _t(2, 40, 2, 64)
    elif case == "out_dtype":
        extra["out"] = _t(2, 4, 64, dtype=torch.float32)
    elif case == "lse_shape":
        extra["lse_out"] = _t(4, 2, dtype=torch.float32)
    elif case == "seqlens_count":
        lens = [50]
    elif case == "heads":
        kc, vc = _t(2, 50, 3, 64), _t(2, 50, 3, 64)
    with pytest.raises(ValueError):
        jlb.bifocal_decode(q, kc, vc, lens, **_PF, **extra)


def test_binding_paged_chunk_fp8_and_quantize_reject_mismatched_tensors():
    import torch
    q = _t(2, 4, 64)
    kp, vp = _t(8, 16, 2, 64), _t(8, 16, 2, 64)
    bt = torch.zeros(1, 8, dtype=torch.int32)  # one row for two sequences
    with pytest.raises(ValueError):
        jlb.bifocal_decode_paged(q, kp, vp, bt, [16, 16], **_PF)
    with pytest.raises(ValueError):  # values of another page size
        jlb.bifocal_decode_paged(q, kp, _t(8, 32, 2, 64), torch.zeros(2, 8, dtype=torch.int32),
                                 [16, 16], **_PF)
    with pytest.raises(ValueError):  # chunk caches with too few rows
        jlb.bifocal_prefill_chunk(_t(10, 4, 64), _t(1, 50, 2, 64), _t(1, 50, 2, 64), [50, 50],
                                  cu_seqlens_q=[0, 5, 10], **_PF)
    with pytest.raises(ValueError):  # chunk of fp32 queries
        jlb.bifocal_prefill_chunk(_t(10, 4, 64, dtype=torch.float32),
                                  _t(1, 50, 2, 64, dtype=torch.float32),
                                  _t(1, 50, 2, 64, dtype=torch.float32), [50], **_PF)
    u8 = torch.zeros(2, 50, 2, 64, dtype=torch.uint8)
    with pytest.raises(ValueError):  # a bf16 cache where codes are expected
        jlb.bifocal_decode_fp8(q, _t(2, 50, 2, 64), u8, [1.0, 1.0], [1.0, 1.0], [50, 50], **_PF)
    with pytest.raises(ValueError):  # fp32 queries on the fp8 path
        jlb.bifocal_decode_fp8(_t(2, 4, 64, dtype=torch.float32), u8, u8, [1.0, 1.0],
                               [1.0, 1.0], [50, 50], **_PF)
    with pytest.raises(ValueError):  # quantize output of the wrong shape
        jlb.kv_quantize_fp8(_t(5, 2, 64), [1.0, 1.0], out=torch.zeros(5, 2, 32, dtype=torch.uint8))
    with pytest.raises(ValueError):  # rope positions of the wrong length
        jlb.rope_apply(_t(5, 2, 64), torch.arange(4), 1e4)


def test_precise_workspaces_cover_every_key():
    """Split precision on every row needs low-part key tiles for every key, so
    its prefill and chunk workspaces are larger; the default ones are unchanged
    by a NULL or default params pointer; a bad precise value is refused."""
    L = jlb.lib()
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    d0, d1 = _params(), _params(precise=1)
    assert L.jl_bifocal_prefill_workspace(131072, 1, 32, 8, 128, 1, None, ctypes.byref(a)) == 0
    assert L.jl_bifocal_prefill_workspace(131072, 1, 32, 8, 128, 1, ctypes.byref(d0),
                                          ctypes.byref(b)) == 0
    assert L.jl_bifocal_prefill_workspace(131072, 1, 32, 8, 128, 1, ctypes.byref(d1),
                                          ctypes.byref(c)) == 0
    assert a.value == b.value and c.value > a.value
    # the low-part tiles of every key: 2 copies x 8 heads x 131072 keys x 128 halves
    assert c.value - a.value >= 2 * 8 * (131072 - 2048) * 128 * 2
    assert L.jl_bifocal_prefill_chunk_workspace(1024, 1, 131072, 32, 8, 128, 1, ctypes.byref(d1),
                                                ctypes.byref(c)) == 0
    assert L.jl_bifocal_prefill_workspace(10, 1, 1, 1, 64, 1, ctypes.byref(_params(precise=3)),
                                          ctypes.byref(c)) == 1


def test_precise_fp8_decode_is_unsupported():
    p = _params(precise=1)
    st = jlb.lib().jl_bifocal_decode_fp8(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, FAKE * 6,
                                         FAKE * 7, FAKE * 9, 1, 1024, 1024, 32, 8, 128,
                                         ctypes.byref(p), FAKE * 8, 1 << 40, None)
    assert st == jlb.JL_ERR_UNSUPPORTED


def test_noalloc_decode_rejects_sizes_beyond_its_scratch():
    """jl_bifocal_decode_noalloc keeps its partials in a 32 MiB static device
    array: a batch whose partials exceed it is refused before any HIP call,
    with the size in the message (fake pointers are never touched)."""
    p = _params()
    st = jlb.lib().jl_bifocal_decode_noalloc(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5,
                                            FAKE * 6, 64, 131072, 131072, 32, 8, 128,
                                            ctypes.byref(p), 1, None)
    assert st == jlb.JL_ERR_WORKSPACE_TOO_SMALL
    assert b"static scratch" in jlb.lib().jl_last_error()
    st = jlb.lib().jl_bifocal_decode_noalloc(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5,
                                            None, 1, 4096, 4096, 32, 8, 128, ctypes.byref(p), 1,
                                            None)
    assert st == jlb.JL_ERR_INVALID_ARGUMENT


def _dec3(**kw):
    a = dict(o=FAKE, lse=FAKE * 2, q=FAKE * 3, kc=FAKE * 4, vc=FAKE * 5, sl=FAKE * 6, B=1,
             max_k=4096, S_max=4096, Hq=32, Hkv=8, d=128, params=_params(), dtype=1,
             ws=FAKE * 8, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    p = a["params"]
    return jlb.lib().jl_bifocal_decode_three_call(
        a["o"], a["lse"], a["q"], a["kc"], a["vc"], a["sl"], a["B"], a["max_k"], a["S_max"],
        a["Hq"], a["Hkv"], a["d"], None if p is None else ctypes.byref(p), a["dtype"], a["ws"],
        a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), 1), (dict(sl=None), 1), (dict(ws=None), 1), (dict(params=None), 1),
    (dict(params=_params(bifocal=0)), 1), (dict(params=_params(bifocal=2)), 1),
    (dict(params=_params(precise=1)), 2), (dict(dtype=0), 2), (dict(B=0), 1),
    (dict(S_max=100), 1), (dict(Hq=30), 1), (dict(Hq=64, Hkv=2), 2), (dict(d=96), 2),
    (dict(ws_bytes=4096), 3), (dict(ws=FAKE * 8 + 8), 1), (dict(o=FAKE * 3), 1),
    (dict(q=FAKE * 3 + 8), 1),
])
def test_three_call_decode_validation(kw, status):
    assert _dec3(**kw) == status


def test_three_call_decode_workspace_query():
    L = jlb.lib()
    n, m = ctypes.c_size_t(), ctypes.c_size_t()
    p = _params()
    assert L.jl_bifocal_decode_three_call_workspace(1, 131072, 32, 8, 128, 1, ctypes.byref(p),
                                                    ctypes.byref(n)) == 0
    # at least the remapped copy of the keys (bf16) and the decode partials
    assert L.jl_bifocal_decode_workspace(1, 131072, 32, 8, 128, 1, ctypes.byref(m)) == 0
    assert n.value >= 131072 * 8 * 128 * 2 + m.value
    assert L.jl_bifocal_decode_three_call_workspace(1, 100, 32, 8, 128, 0, ctypes.byref(p),
                                                    ctypes.byref(n)) == 2
    assert L.jl_bifocal_decode_three_call_workspace(1, 100, 32, 8, 128, 1, None,
                                                    ctypes.byref(n)) == 1

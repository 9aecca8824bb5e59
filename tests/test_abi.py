"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments before touching the GPU (runs on CPU; no kernel is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qkvfa.h")
LIB = os.path.join(ROOT, "quantized_kv_flashattention_amd", "libqkvfa.so")


@pytest.fixture(scope="module")
def lib():
    assert os.path.exists(LIB), "libqkvfa.so is not built (conftest builds it when missing)"
    L = ctypes.CDLL(LIB)
    i64, vp, f32, ci, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    L.qkv_quantize_append.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
    L.qkv_quantize_append_kv.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
    L.qkv_decode.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, f32, ci, vp, vp, vp, sz, vp]
    L.qkv_prefill.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, f32, ci, vp, vp, vp]
    L.qkv_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, f32, ci,
                                    vp, vp, vp, sz, vp]
    L.qkv_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64,
                                   i64, i64, f32, ci, vp, vp, vp, sz, vp]
    L.qkv_buffer_scale.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp]
    L.qkv_buffer_flush.argtypes = [vp, vp, vp, vp, i64, i64, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp]
    L.qkv_decode_buffered.argtypes = [vp] * 11 + [i64] * 10 + [f32, ci, vp, vp, vp, sz, vp]
    L.qkv_decode_buffered_workspace_bytes.restype = sz
    L.qkv_decode_buffered_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, ci]
    L.qkv_last_error.restype = ctypes.c_char_p
    L.qkv_status_string.restype = ctypes.c_char_p
    L.qkv_decode_workspace_bytes.restype = sz
    L.qkv_decode_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, ci]
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qkv_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) >= {"qkv_quantize_append", "qkv_decode", "qkv_decode_append", "qkv_decode_paged",
                          "qkv_buffer_scale", "qkv_buffer_flush", "qkv_decode_buffered",
                          "qkv_decode_buffered_workspace_bytes", "qkv_prefill",
                          "qkv_quantize_append_kv", "qkv_decode_workspace_bytes",
                          "qkv_decode_auto_splits", "qkv_last_error", "qkv_status_string", "qkv_version",
                          "qkv_quantize_append_kv_bits", "qkv_decode_bits", "qkv_quantize_append_kv_asym",
                          "qkv_decode_asym", "qkv_quantize_append_kv_heads", "qkv_decode_heads",
                          "qkv_prefill_bits", "qkv_prefill_asym", "qkv_prefill_heads"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.qkv_status_string(0) == b"ok"
    assert lib.qkv_status_string(3) == b"workspace too small"
    assert lib.qkv_version() == 100


P = 16  # a fake, 16-byte aligned non-null address: never dereferenced on these paths


def _qa(lib, **kw):
    a = dict(src=P, codes=P, scales=P, B=1, Hkv=1, T=4, D=128, C=8, pos=0)
    a.update(kw)
    return lib.qkv_quantize_append(a["src"], a["codes"], a["scales"], a["B"], a["Hkv"], a["T"], a["D"],
                                   a["C"], a["pos"], None)


def test_quantize_append_argument_errors(lib):
    assert _qa(lib, D=96) == 2
    assert _qa(lib, pos=5) == 1                 # pos + T > C
    assert b"pos" in lib.qkv_last_error()
    assert _qa(lib, pos=-1) == 1
    assert _qa(lib, B=0) == 1
    assert _qa(lib, src=None) == 1
    assert _qa(lib, src=P + 4) == 1             # misaligned
    assert _qa(lib, scales=P + 1) == 1
    assert b"misaligned" in lib.qkv_last_error()
    assert _qa(lib, T=0, src=None) == 0         # nothing to do: ok, nothing enqueued


def _dec(lib, **kw):
    a = dict(q=P, kc=P, ks=P, vc=P, vs=P, B=1, Hq=4, Hkv=2, Sq=1, L=100, C=128, D=128, scale=0.1, ns=0,
             out=P, lse=None, ws=None, wsb=0)
    a.update(kw)
    return lib.qkv_decode(a["q"], a["kc"], a["ks"], a["vc"], a["vs"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["L"],
                          a["C"], a["D"], a["scale"], a["ns"], a["out"], a["lse"], a["ws"], a["wsb"], None)


def test_decode_argument_errors(lib):
    assert _dec(lib, D=80) == 2
    assert _dec(lib, Hq=3) == 1                 # Hq % Hkv
    assert _dec(lib, L=0) == 1
    assert _dec(lib, L=129) == 1                # kv_len > C
    assert _dec(lib, Sq=33) == 2                # G * Sq > 64
    assert _dec(lib, q=None) == 1
    assert _dec(lib, out=P + 8) == 1
    assert _dec(lib, ns=-1) == 1
    assert _dec(lib, ns=2000) == 1
    assert _dec(lib, ns=2) == 3                 # needs a workspace
    assert b"workspace" in lib.qkv_last_error()
    assert _dec(lib, ns=2, ws=P, wsb=10) == 3
    assert _dec(lib, B=65535, Hkv=256, Hq=256, L=64, C=64, D=64, ns=1) == 2   # grid beyond 2^32 threads
    assert b"workgroups" in lib.qkv_last_error()


def test_decode_workspace_size(lib):
    assert lib.qkv_decode_workspace_bytes(1, 4, 2, 1, 100, 128, 1) == 0
    n = lib.qkv_decode_workspace_bytes(1, 4, 2, 1, 100, 128, 2)
    assert n >= 4 * 2 * 128 * 4 + 4 * 2 * 4
    assert lib.qkv_decode_workspace_bytes(1, 4, 2, 1, 100, 96, 2) == 0


def _pre(lib, **kw):
    a = dict(q=P, kc=P, ks=P, vc=P, vs=P, B=1, Hq=4, Hkv=2, Sq=10, L=100, C=128, D=64, scale=0.1, causal=1,
             out=P, lse=None)
    a.update(kw)
    return lib.qkv_prefill(a["q"], a["kc"], a["ks"], a["vc"], a["vs"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["L"],
                           a["C"], a["D"], a["scale"], a["causal"], a["out"], a["lse"], None)


def test_prefill_argument_errors(lib):
    assert _pre(lib, Sq=101) == 1               # causal needs Sq <= kv_len
    assert _pre(lib, causal=2) == 1
    assert _pre(lib, D=32) == 2
    assert _pre(lib, Hkv=3) == 1
    assert _pre(lib, lse=P + 2) == 1
    assert _pre(lib, kc=P + 8) == 1


def test_quantize_append_kv_argument_errors(lib):
    f = lambda **kw: lib.qkv_quantize_append_kv(*(kw.get(n, P) for n in ("ks_", "vs_", "kc", "kss", "vc", "vss")),
                                                kw.get("B", 1), 1, kw.get("T", 4), kw.get("D", 64), 8,
                                                kw.get("pos", 0), None)
    assert f(D=32) == 2
    assert f(pos=6) == 1
    assert f(vs_=None) == 1
    assert f(kc=P + 2) == 1
    assert f(B=0) == 1
    assert f(T=0, vs_=None) == 0


def _dapp(lib, **kw):
    a = dict(q=P, kn=P, vn=P, kc=P, ks=P, vc=P, vs=P, B=1, Hq=4, Hkv=2, Sq=1, pos=99, n=1, C=128, D=128,
             scale=0.1, ns=0, out=P, lse=None, ws=None, wsb=0)
    a.update(kw)
    return lib.qkv_decode_append(a["q"], a["kn"], a["vn"], a["kc"], a["ks"], a["vc"], a["vs"], a["B"], a["Hq"],
                                 a["Hkv"], a["Sq"], a["pos"], a["n"], a["C"], a["D"], a["scale"], a["ns"],
                                 a["out"], a["lse"], a["ws"], a["wsb"], None)


def test_decode_append_argument_errors(lib):
    assert _dapp(lib, kn=None) == 1
    assert b"new-row" in lib.qkv_last_error()
    assert _dapp(lib, vn=P + 4) == 1            # misaligned new rows
    assert _dapp(lib, n=0) == 2
    assert _dapp(lib, n=65) == 2
    assert _dapp(lib, pos=-1) == 1
    assert _dapp(lib, pos=128) == 1             # pos + n_new > C
    assert _dapp(lib, D=80) == 2
    assert _dapp(lib, Sq=33) == 2               # G * Sq > 64
    assert _dapp(lib, ns=2) == 3                # needs a workspace
    assert b"qkv_decode_append" in lib.qkv_last_error()
    assert _dapp(lib, q=None) == 1


def _paged(lib, **kw):
    a = dict(q=P, kn=None, vn=None, kc=P, ks=P, vc=P, vs=P, bt=P, lens=P, B=2, Hq=4, Hkv=2, Sq=1, n=0,
             maxlen=100, ps=64, mp=4, np_=16, D=128, scale=0.1, ns=0, out=P, lse=None, ws=None, wsb=0)
    a.update(kw)
    return lib.qkv_decode_paged(a["q"], a["kn"], a["vn"], a["kc"], a["ks"], a["vc"], a["vs"], a["bt"], a["lens"],
                                a["B"], a["Hq"], a["Hkv"], a["Sq"], a["n"], a["maxlen"], a["ps"], a["mp"],
                                a["np_"], a["D"], a["scale"], a["ns"], a["out"], a["lse"], a["ws"], a["wsb"],
                                None)


def test_decode_paged_argument_errors(lib):
    assert _paged(lib, ps=48) == 2              # a page must hold whole 32-row chunks
    assert b"multiple of 32" in lib.qkv_last_error()
    assert _paged(lib, ps=0) == 1
    assert _paged(lib, mp=0) == 1
    assert _paged(lib, bt=None, mp=2) == 1      # without a table: one page per sequence
    assert _paged(lib, bt=None, mp=1, np_=1) == 1   # ... and at least B pages
    assert b"page b" in lib.qkv_last_error()
    assert _paged(lib, bt=P + 2) == 1           # misaligned table
    assert _paged(lib, lens=P + 1) == 1         # misaligned lengths
    assert _paged(lib, n=65) == 2
    assert _paged(lib, n=-1) == 2
    assert _paged(lib, n=1) == 1                # new rows but no k_new / v_new
    assert b"new-row" in lib.qkv_last_error()
    assert _paged(lib, n=1, kn=P, vn=P + 4) == 1
    assert _paged(lib, maxlen=257) == 1         # beyond max_pages * page_size
    assert _paged(lib, maxlen=0) == 1
    assert _paged(lib, n=3, kn=P, vn=P, maxlen=2) == 1   # max_kv_len < n_new
    assert _paged(lib, D=96) == 2
    assert _paged(lib, Sq=33) == 2              # G * Sq > 64
    assert _paged(lib, q=None) == 1
    assert _paged(lib, ps=1 << 20, mp=1 << 12) == 2      # capacity beyond 2^31 rows
    assert _paged(lib, maxlen=256, ns=3) == 3   # needs a workspace
    assert b"qkv_decode_paged" in lib.qkv_last_error()


def test_buffer_scale_argument_errors(lib):
    f = lambda **kw: lib.qkv_buffer_scale(kw.get("ks", P), kw.get("vs", P), kw.get("B", 1), 1, kw.get("L", 4),
                                          kw.get("C", 8), kw.get("k8", P), kw.get("v8", P), None)
    assert f(L=9) == 1
    assert f(L=-1) == 1
    assert f(ks=None) == 1
    assert f(k8=P + 2) == 1
    assert f(B=0) == 1


def test_buffer_flush_argument_errors(lib):
    def f(**kw):
        a = dict(kb=P, vb=P, k8=P, v8=P, rows=64, T=10, kc=P, ks=P, vc=P, vs=P, B=1, Hkv=1, D=128, C=100, pos=0)
        a.update(kw)
        return lib.qkv_buffer_flush(a["kb"], a["vb"], a["k8"], a["v8"], a["rows"], a["T"], a["kc"], a["ks"],
                                    a["vc"], a["vs"], a["B"], a["Hkv"], a["D"], a["C"], a["pos"], None)
    assert f(rows=65) == 1
    assert f(T=65, rows=64) == 1
    assert f(pos=91) == 1
    assert f(D=96) == 2
    assert f(kb=None) == 1
    assert f(vb=P + 8) == 1
    assert f(T=0, kb=None) == 0        # nothing to do


def _dbuf(lib, **kw):
    a = dict(q=P, kn=P, vn=P, kc=P, ks=P, vc=P, vs=P, kb=P, vb=P, k8=P, v8=P, B=1, Hq=4, Hkv=2, Sq=1, L=100,
             C=128, rows=64, blen=3, n=1, D=128, scale=0.1, ns=0, out=P, lse=None, ws=None, wsb=0)
    a.update(kw)
    return lib.qkv_decode_buffered(a["q"], a["kn"], a["vn"], a["kc"], a["ks"], a["vc"], a["vs"], a["kb"], a["vb"],
                                   a["k8"], a["v8"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["L"], a["C"], a["rows"],
                                   a["blen"], a["n"], a["D"], a["scale"], a["ns"], a["out"], a["lse"], a["ws"],
                                   a["wsb"], None)


def test_decode_buffered_argument_errors(lib):
    assert _dbuf(lib, rows=65) == 2
    assert _dbuf(lib, blen=64, n=1) == 1        # more rows than the buffer holds
    assert _dbuf(lib, blen=-1) == 1
    assert _dbuf(lib, L=129) == 1
    assert _dbuf(lib, L=0, blen=0, n=0) == 1    # nothing to attend
    assert _dbuf(lib, kb=None) == 1
    assert b"buffer" in lib.qkv_last_error()
    assert _dbuf(lib, k8=P + 1) == 1
    assert _dbuf(lib, kn=None) == 1
    assert _dbuf(lib, vn=P + 4) == 1
    assert _dbuf(lib, D=80) == 2
    assert _dbuf(lib, Sq=33) == 2
    assert _dbuf(lib, ns=3) == 3                # body splits + the buffer split need a workspace
    assert b"qkv_decode_buffered" in lib.qkv_last_error()
    assert _dbuf(lib, q=None) == 1


def test_decode_buffered_workspace_size(lib):
    # no cache rows: the buffer split alone writes the output directly
    assert lib.qkv_decode_buffered_workspace_bytes(1, 4, 2, 1, 0, 128, 0) == 0
    # one cache split + the buffer split
    n = lib.qkv_decode_buffered_workspace_bytes(1, 4, 2, 1, 100, 128, 1)
    assert n >= 4 * 2 * 128 * 4


def test_lowbit_argument_errors(lib):
    i64, vp, f32, ci, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    lib.qkv_quantize_append_kv_bits.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, vp]
    lib.qkv_decode_bits.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ci, f32, ci,
                                    vp, vp, vp, sz, vp]
    qb = lambda **kw: lib.qkv_quantize_append_kv_bits(P, P, P, P, P, P, 1, 1, kw.get("T", 4), kw.get("D", 64), 8,
                                                      kw.get("pos", 0), kw.get("bits", 2), None)
    assert qb(bits=5) == 2
    assert qb(bits=1) == 2
    assert qb(D=96) == 2
    assert qb(pos=5) == 1
    assert qb(T=0) == 0
    db = lambda **kw: lib.qkv_decode_bits(P, P, P, P, P, 1, 4, 2, 1, kw.get("L", 100), 128, kw.get("D", 128),
                                          kw.get("bits", 3), 0.1, kw.get("ns", 0), P, None, None, 0, None)
    assert db(bits=8) == 2
    assert db(D=80) == 2
    assert db(L=129) == 1
    assert db(ns=2) == 3
    assert b"qkv_decode_bits" in lib.qkv_last_error()


def test_asym_argument_errors(lib):
    i64, vp, f32, ci, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    lib.qkv_quantize_append_kv_asym.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, vp]
    lib.qkv_decode_asym.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ci, f32, ci,
                                    vp, vp, vp, sz, vp]
    qa = lambda **kw: lib.qkv_quantize_append_kv_asym(P, P, P, kw.get("kp", P), P, P, 1, 1, kw.get("T", 4),
                                                      kw.get("D", 64), 8, kw.get("pos", 0), kw.get("g", 32), None)
    assert qa(g=16) == 2
    assert qa(g=128) == 2        # group larger than the head dim
    assert qa(g=48) == 2
    assert qa(D=96) == 2
    assert qa(pos=5) == 1
    assert qa(kp=None) == 1
    assert qa(kp=P + 2) == 1     # parameter words are 4-byte aligned
    assert qa(T=0) == 0
    assert b"qkv_quantize_append_kv_asym" in lib.qkv_last_error()
    da = lambda **kw: lib.qkv_decode_asym(P, P, kw.get("kp", P), P, P, 1, 4, 2, 1, kw.get("L", 100), 128,
                                          kw.get("D", 128), kw.get("g", 64), 0.1, kw.get("ns", 0), P, None, None, 0,
                                          None)
    assert da(g=256) == 2
    assert da(D=64, g=128) == 2
    assert da(D=80) == 2
    assert da(L=129) == 1
    assert da(kp=None) == 1
    assert da(kp=P + 2) == 1
    assert da(ns=2) == 3         # two splits need a workspace
    assert b"qkv_decode_asym" in lib.qkv_last_error()


def test_head_map_argument_errors(lib):
    i64, vp, f32, ci, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    lib.qkv_quantize_append_kv_heads.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci,
                                                 vp]
    lib.qkv_decode_heads.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, ci, f32, ci,
                                     vp, vp, vp, sz, vp]
    qh = lambda **kw: lib.qkv_quantize_append_kv_heads(P, P, kw.get("heads", P), kw.get("hs", 2), P, P, P, P, 1,
                                                       kw.get("H", 4), kw.get("T", 4), 64, 8, kw.get("pos", 0),
                                                       kw.get("bits", 4), None)
    assert qh(bits=5) == 2
    assert qh(hs=0) == 1
    assert qh(hs=5) == 1          # more heads than the layer has
    assert qh(heads=None) == 1
    assert qh(heads=P + 2) == 1
    assert qh(pos=6) == 1
    assert qh(T=0) == 0
    assert b"qkv_quantize_append_kv_heads" in lib.qkv_last_error()
    dh = lambda **kw: lib.qkv_decode_heads(P, P, P, P, P, kw.get("heads", P), kw.get("hs", 2), 1, 8, 4, 1,
                                           kw.get("L", 100), 128, 128, kw.get("bits", 2), 0.1, kw.get("ns", 0), P,
                                           None, None, 0, None)
    assert dh(bits=1) == 2
    assert dh(hs=0) == 1
    assert dh(hs=5) == 1
    assert dh(heads=None) == 1
    assert dh(L=129) == 1
    assert dh(ns=2) == 3
    assert b"qkv_decode_heads" in lib.qkv_last_error()


def test_prefill_bits_argument_errors(lib):
    i64, vp, f32, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    lib.qkv_prefill_bits.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ci, f32, ci, vp, vp, vp]
    pb = lambda **kw: lib.qkv_prefill_bits(P, P, P, P, P, 1, 4, 2, kw.get("Sq", 10), kw.get("L", 100), 128,
                                           kw.get("D", 64), kw.get("bits", 2), 0.1, kw.get("causal", 1), P, None,
                                           None)
    assert pb(bits=1) == 2
    assert pb(bits=8) == 2
    assert pb(D=96) == 2
    assert pb(causal=2) == 1
    assert pb(Sq=101) == 1        # causal needs Sq <= kv_len
    assert pb(L=129) == 1
    assert b"qkv_prefill_bits" in lib.qkv_last_error()


def test_prefill_asym_argument_errors(lib):
    i64, vp, f32, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    lib.qkv_prefill_asym.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ci, f32, ci, vp, vp, vp]
    pa = lambda **kw: lib.qkv_prefill_asym(P, P, kw.get("kp", P), P, P, 1, 4, 2, kw.get("Sq", 10), kw.get("L", 100),
                                           128, kw.get("D", 128), kw.get("g", 32), 0.1, kw.get("causal", 1), P, None,
                                           None)
    assert pa(g=16) == 2
    assert pa(D=64, g=128) == 2   # group larger than the head dim
    assert pa(D=96) == 2
    assert pa(kp=None) == 1
    assert pa(kp=P + 4) == 1      # four words per row: 16-byte aligned
    assert pa(g=64, kp=P + 4) == 1   # two words: 8-byte aligned
    assert pa(causal=2) == 1
    assert pa(Sq=101) == 1        # causal needs Sq <= kv_len
    assert pa(L=129) == 1
    assert b"qkv_prefill_asym" in lib.qkv_last_error()


def test_prefill_heads_argument_errors(lib):
    i64, vp, f32, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    lib.qkv_prefill_heads.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, ci, f32, ci,
                                      vp, vp, vp]
    ph = lambda **kw: lib.qkv_prefill_heads(P, P, P, P, P, kw.get("heads", P), kw.get("hs", 2), 1, 8, 4,
                                            kw.get("Sq", 10), kw.get("L", 100), 128, 128, kw.get("bits", 2), 0.1,
                                            kw.get("causal", 1), P, None, None)
    assert ph(bits=1) == 2
    assert ph(hs=0) == 1
    assert ph(hs=5) == 1          # more heads than the layer has
    assert ph(heads=None) == 1
    assert ph(heads=P + 2) == 1
    assert ph(causal=2) == 1
    assert ph(Sq=101) == 1        # causal needs Sq <= kv_len
    assert ph(L=129) == 1
    assert b"qkv_prefill_heads" in lib.qkv_last_error()


def test_decode_noalloc_argument_errors(lib):
    lib.qkv_decode_noalloc.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 7 + \
        [ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]

    def nd(**kw):
        a = dict(B=1, Hq=4, Hkv=2, Sq=1, L=100, C=128, D=128, ns=0, q=P, out=P)
        a.update(kw)
        return lib.qkv_decode_noalloc(a["q"], P, P, P, P, a["B"], a["Hq"], a["Hkv"], a["Sq"], a["L"], a["C"],
                                      a["D"], 0.1, a["ns"], a["out"], None, None)
    assert nd(D=80) == 2
    assert nd(q=None) == 1
    assert nd(ns=-1) == 1
    # more (batch, KV head) tickets than the static scratch holds
    assert nd(B=4097, Hq=1, Hkv=1, ns=2) == 3
    assert b"static scratch" in lib.qkv_last_error()
    # 1024 rows x 64 splits x (128 + 1) x 4 bytes of partials: past 16 MiB
    assert nd(B=16, Hq=64, Hkv=1, L=131072, C=131072, ns=64) == 3
    assert b"static scratch" in lib.qkv_last_error()


BENCH_HEADER = os.path.join(ROOT, "include", "qkvfa_bench.h")
BENCH_LIB = os.path.join(ROOT, "quantized_kv_flashattention_amd", "libqkvfa_bench.so")


def test_bench_helper_exports_and_argument_errors():
    L = ctypes.CDLL(BENCH_LIB)
    text = re.sub(r"/\*.*?\*/", "", open(BENCH_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(qkvb_[a-z_0-9]+)\s*\(", text)))
    assert names == ["qkvb_stream_read"]
    for n in names:
        assert hasattr(L, n), n
    f = L.qkvb_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert f(None, 16, P, 1, None) == 1
    assert f(P, 17, P, 1, None) == 1          # not a multiple of 16
    assert f(P + 4, 16, P, 1, None) == 1      # misaligned
    assert f(P, 16, P, 0, None) == 1
    assert f(P, 16, None, 1, None) == 1


TRACE_HEADER = os.path.join(ROOT, "include", "qkvfa_trace.h")
TRACE_LIB = os.path.join(ROOT, "quantized_kv_flashattention_amd", "libqkvfa_trace.so")


def test_trace_build_exports_the_abi_and_its_reader():
    """The measurement build (decode phase timestamps) exports every call of
    qkvfa.h and qkv_trace_read; bad arguments fail before any device work."""
    if not os.path.exists(TRACE_LIB):
        pytest.skip("libqkvfa_trace.so not built")
    tl = ctypes.CDLL(TRACE_LIB)
    for n in declared_functions():
        assert hasattr(tl, n), n
    text = re.sub(r"/\*.*?\*/", "", open(TRACE_HEADER).read(), flags=re.S)
    assert re.findall(r"\b(qkv_[a-z_0-9]+)\s*\(", text) == ["qkv_trace_read"]
    tl.qkv_trace_read.restype = ctypes.c_int
    tl.qkv_trace_read.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    assert tl.qkv_trace_read(None, 4) == 1                     # QKV_ERR_INVALID_ARG
    buf = (ctypes.c_uint64 * 16)()
    assert tl.qkv_trace_read(ctypes.addressof(buf), -1) == 1
    # the plain library has no trace reader
    assert not hasattr(ctypes.CDLL(os.path.join(ROOT, "quantized_kv_flashattention_amd", "libqkvfa.so")),
                       "qkv_trace_read")

"""int4-KV FlashAttention for AMD MI355X (gfx950): Python binding of libqkvfa.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libqkvfa.so`` (built in-tree by ``build.py``); PyTorch provides
device memory and the current stream.  There is no CPU or eager fallback:
importing this package fails if the library is missing.

Tensors (all on one CUDA/HIP device, contiguous):

* cache: ``k_codes``/``v_codes`` uint8 ``[B, Hkv, C, D/2]`` and
  ``k_scales``/``v_scales`` float16 ``[B, Hkv, C]`` (one scale per token and
  KV head); :class:`KVCache` allocates them,
* ``q`` bfloat16 ``[B, Hq, Sq, D]``, outputs float32 ``[B, Hq, Sq, D]`` and,
  on request, the natural-log LSE float32 ``[B, Hq, Sq]``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

import torch

__all__ = [
    "QKVError",
    "KVCache",
    "quantize_append",
    "quantize_append_kv",
    "decode",
    "decode_noalloc",
    "decode_append",
    "decode_paged",
    "DecodeBuffer",
    "buffer_scale",
    "buffer_flush",
    "decode_buffered",
    "decode_buffered_workspace_bytes",
    "quantize_append_kv_heads",
    "decode_heads",
    "decode_mixed",
    "prefill_heads",
    "prefill_mixed",
    "AsymKVCache",
    "quantize_append_kv_asym",
    "decode_asym",
    "prefill_asym",
    "prefill",
    "decode_workspace_bytes",
    "decode_auto_splits",
    "version",
    "library_path",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG_DIR, "libqkvfa.so")


class QKVError(RuntimeError):
    """A libqkvfa call returned a nonzero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python quantized_kv_flashattention_amd/build.py`")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, vp, f32, ci, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    lib.qkv_status_string.restype = ctypes.c_char_p
    lib.qkv_status_string.argtypes = [ci]
    lib.qkv_last_error.restype = ctypes.c_char_p
    lib.qkv_last_error.argtypes = []
    lib.qkv_version.restype = ci
    lib.qkv_version.argtypes = []
    lib.qkv_quantize_append.restype = ci
    lib.qkv_quantize_append.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
    lib.qkv_quantize_append_kv.restype = ci
    lib.qkv_quantize_append_kv.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
    lib.qkv_decode_workspace_bytes.restype = sz
    lib.qkv_decode_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, ci]
    lib.qkv_decode_auto_splits.restype = ci
    lib.qkv_decode_auto_splits.argtypes = [i64, i64, i64, i64, i64, i64]
    lib.qkv_decode.restype = ci
    lib.qkv_decode.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, f32, ci,
                               vp, vp, vp, sz, vp]
    lib.qkv_decode_noalloc.restype = ci
    lib.qkv_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, f32, ci,
                                       vp, vp, vp]
    lib.qkv_decode_append.restype = ci
    lib.qkv_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64,
                                      f32, ci, vp, vp, vp, sz, vp]
    lib.qkv_prefill.restype = ci
    lib.qkv_decode_paged.restype = ci
    lib.qkv_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                     i64, i64, i64, f32, ci, vp, vp, vp, sz, vp]
    lib.qkv_buffer_scale.restype = ci
    lib.qkv_buffer_scale.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp]
    lib.qkv_buffer_flush.restype = ci
    lib.qkv_buffer_flush.argtypes = [vp, vp, vp, vp, i64, i64, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp]
    lib.qkv_decode_buffered_workspace_bytes.restype = sz
    lib.qkv_decode_buffered_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, ci]
    lib.qkv_decode_buffered.restype = ci
    lib.qkv_decode_buffered.argtypes = [vp] * 11 + [i64] * 10 + [f32, ci, vp, vp, vp, sz, vp]
    lib.qkv_quantize_append_kv_bits.restype = ci
    lib.qkv_quantize_append_kv_bits.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, vp]
    lib.qkv_decode_bits.restype = ci
    lib.qkv_decode_bits.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ci, f32, ci,
                                    vp, vp, vp, sz, vp]
    lib.qkv_prefill.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, f32, ci,
                                vp, vp, vp]
    lib.qkv_quantize_append_kv_asym.restype = ci
    lib.qkv_quantize_append_kv_asym.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, vp]
    lib.qkv_quantize_append_kv_heads.restype = ci
    lib.qkv_quantize_append_kv_heads.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci,
                                                 vp]
    lib.qkv_decode_heads.restype = ci
    lib.qkv_decode_heads.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, ci, f32, ci,
                                     vp, vp, vp, sz, vp]
    lib.qkv_prefill_bits.restype = ci
    lib.qkv_prefill_bits.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ci, f32, ci, vp, vp, vp]
    lib.qkv_prefill_heads.restype = ci
    lib.qkv_prefill_heads.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, ci, f32, ci,
                                      vp, vp, vp]
    lib.qkv_prefill_asym.restype = ci
    lib.qkv_prefill_asym.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ci, f32, ci, vp, vp, vp]
    lib.qkv_decode_asym.restype = ci
    lib.qkv_decode_asym.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ci, f32, ci,
                                    vp, vp, vp, sz, vp]
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def version() -> int:
    return int(_lib.qkv_version())


def _check(status: int):
    if status != 0:
        raise QKVError(status, _lib.qkv_last_error().decode(errors="replace"))


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _req(t: torch.Tensor, name: str, dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


@dataclasses.dataclass
class KVCache:
    """Caller-owned int4 KV cache of one layer."""

    k_codes: torch.Tensor   # uint8 [B, Hkv, C, D/2]
    k_scales: torch.Tensor  # float16 [B, Hkv, C]
    v_codes: torch.Tensor
    v_scales: torch.Tensor

    @staticmethod
    def empty(B: int, Hkv: int, C: int, D: int, device="cuda", bits: int = 4) -> "KVCache":
        """Cache of ``bits``-bit rows (``D * bits / 8`` bytes of codes per row)."""
        mk = lambda: torch.empty((B, Hkv, C, D * bits // 8), dtype=torch.uint8, device=device)
        ms = lambda: torch.empty((B, Hkv, C), dtype=torch.float16, device=device)
        return KVCache(mk(), ms(), mk(), ms())

    @property
    def shape(self):
        B, Hkv, C, half = self.k_codes.shape
        return B, Hkv, C, 2 * half

    def tensors(self):
        return self.k_codes, self.k_scales, self.v_codes, self.v_scales


def quantize_append(src: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, pos: int):
    """Quantize fp32 rows ``src [B, Hkv, T, D]`` into cache rows ``[pos, pos+T)``."""
    _req(src, "src", torch.float32, 4)
    _req(codes, "codes", torch.uint8, 4)
    _req(scales, "scales", torch.float16, 3)
    B, Hkv, T, D = src.shape
    if codes.shape[:2] != (B, Hkv) or codes.shape[3] * 2 != D or scales.shape != codes.shape[:3]:
        raise ValueError("cache shape does not match src")
    if src.device != codes.device or src.device != scales.device:
        raise ValueError("all tensors must be on one device")
    C = codes.shape[2]
    _check(_lib.qkv_quantize_append(_ptr(src), _ptr(codes), _ptr(scales), B, Hkv, T, D, C, int(pos),
                                    _stream(src)))


def quantize_append_kv(k_src: torch.Tensor, v_src: torch.Tensor, cache: "KVCache", pos: int, bits: int = 4):
    """Quantize new K and V rows ``[B, Hkv, T, D]`` into cache rows ``[pos, pos+T)`` in one launch
    (``bits`` = 2, 3 or 4; the cache's code rows hold ``D * bits / 8`` bytes)."""
    _req(k_src, "k_src", torch.float32, 4)
    _req(v_src, "v_src", torch.float32, 4)
    if k_src.shape != v_src.shape or k_src.device != v_src.device:
        raise ValueError("k_src and v_src must have one shape and device")
    kc, ks, vc, vs = cache.tensors() if isinstance(cache, KVCache) else tuple(cache)
    for name, t, dt, nd in (("k_codes", kc, torch.uint8, 4), ("k_scales", ks, torch.float16, 3),
                            ("v_codes", vc, torch.uint8, 4), ("v_scales", vs, torch.float16, 3)):
        _req(t, name, dt, nd)
        if t.device != k_src.device:
            raise ValueError("all tensors must be on one device")
    B, Hkv, T, D = k_src.shape
    if kc.shape[:2] != (B, Hkv) or kc.shape[3] * 8 != D * bits or vc.shape != kc.shape or \
            ks.shape != kc.shape[:3] or vs.shape != ks.shape:
        raise ValueError("cache shape does not match src")
    if bits == 4:
        _check(_lib.qkv_quantize_append_kv(_ptr(k_src), _ptr(v_src), _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs),
                                           B, Hkv, T, D, kc.shape[2], int(pos), _stream(k_src)))
    else:
        _check(_lib.qkv_quantize_append_kv_bits(_ptr(k_src), _ptr(v_src), _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs),
                                                B, Hkv, T, D, kc.shape[2], int(pos), int(bits), _stream(k_src)))


def _attn_args(q, cache_tensors, kv_len, bits=4):
    _req(q, "q", torch.bfloat16, 4)
    kc, ks, vc, vs = cache_tensors
    for name, t, dt, nd in (("k_codes", kc, torch.uint8, 4), ("k_scales", ks, torch.float16, 3),
                            ("v_codes", vc, torch.uint8, 4), ("v_scales", vs, torch.float16, 3)):
        _req(t, name, dt, nd)
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")
    B, Hq, Sq, D = q.shape
    Bk, Hkv, C, rowb = kc.shape
    if Bk != B or rowb * 8 != D * bits or vc.shape != kc.shape or ks.shape != (B, Hkv, C) or vs.shape != ks.shape:
        raise ValueError("cache shape does not match q")
    return B, Hq, Hkv, Sq, int(kv_len), C, D


def _outputs(q, out, lse, return_lse):
    """Allocate or check ``out [B, Hq, Sq, D]`` fp32 and (on request) ``lse [B, Hq, Sq]``."""
    B, Hq, Sq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=torch.float32, device=q.device)
    else:
        _req(out, "out", torch.float32, 4)
        if out.shape != q.shape or out.device != q.device:
            raise ValueError("out must have q's shape and device")
    if lse is not None:
        _req(lse, "lse", torch.float32, 3)
        if lse.shape != (B, Hq, Sq) or lse.device != q.device:
            raise ValueError("lse must be [B, Hq, Sq] on q's device")
    elif return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    return out, lse


def _scale(softmax_scale, D):
    return float(1.0 / math.sqrt(D)) if softmax_scale is None else float(softmax_scale)


def decode_workspace_bytes(B, Hq, Hkv, Sq, kv_len, D, num_splits=0) -> int:
    return int(_lib.qkv_decode_workspace_bytes(B, Hq, Hkv, Sq, kv_len, D, num_splits))


def decode_auto_splits(B, Hq, Hkv, Sq, kv_len, D) -> int:
    return int(_lib.qkv_decode_auto_splits(B, Hq, Hkv, Sq, kv_len, D))


_WORKSPACES = {}


def _workspace(device, units, nbytes):
    """A zero-initialised decode workspace per (device, B*Hkv), grown on demand.

    Its ticket counters sit at offset 0 and the kernels return them to zero
    after every call, so it is reused as is by every call with the same
    B*Hkv.  Calls on different streams must not share it: pass an explicit
    zeroed ``workspace`` tensor for concurrent decodes.
    """
    key = (device.type, device.index, int(units))
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


def decode(q, cache, kv_len, softmax_scale=None, num_splits=0, return_lse=False, out=None,
           lse=None, workspace=None, bits=4):
    """Decode attention of ``q [B, Hq, Sq, D]`` over cache rows ``[0, kv_len)`` (no mask);
    ``bits`` = 2, 3 or 4 is the width of the cache's codes."""
    tensors = cache.tensors() if isinstance(cache, KVCache) else tuple(cache)
    B, Hq, Hkv, Sq, kv_len, C, D = _attn_args(q, tensors, kv_len, bits)
    out, lse = _outputs(q, out, lse, return_lse)
    need = decode_workspace_bytes(B, Hq, Hkv, Sq, kv_len, D, num_splits)
    if workspace is None and need > 0:
        workspace = _workspace(q.device, B * Hkv, need)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    kc, ks, vc, vs = tensors
    if bits == 4:
        _check(_lib.qkv_decode(_ptr(q), _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs), B, Hq, Hkv, Sq, kv_len,
                               C, D, _scale(softmax_scale, D), int(num_splits), _ptr(out), _ptr(lse),
                               _ptr(workspace), ws_bytes, _stream(q)))
    else:
        _check(_lib.qkv_decode_bits(_ptr(q), _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs), B, Hq, Hkv, Sq, kv_len,
                                    C, D, int(bits), _scale(softmax_scale, D), int(num_splits), _ptr(out),
                                    _ptr(lse), _ptr(workspace), ws_bytes, _stream(q)))
    return (out, lse) if return_lse else out


def decode_noalloc(q, cache, kv_len, softmax_scale=None, num_splits=0, return_lse=False, out=None, lse=None):
    """``decode`` (int4 cache) through ``qkv_decode_noalloc``: no workspace; the library's
    static per-device scratch holds the split partials.  ``out``/``lse`` given, it
    allocates nothing."""
    tensors = cache.tensors() if isinstance(cache, KVCache) else tuple(cache)
    B, Hq, Hkv, Sq, kv_len, C, D = _attn_args(q, tensors, kv_len, 4)
    out, lse = _outputs(q, out, lse, return_lse)
    kc, ks, vc, vs = tensors
    _check(_lib.qkv_decode_noalloc(_ptr(q), _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs), B, Hq, Hkv, Sq, kv_len,
                                   C, D, _scale(softmax_scale, D), int(num_splits), _ptr(out), _ptr(lse),
                                   _stream(q)))
    return (out, lse) if return_lse else out


def _heads_arg(kv_heads, device):
    _req(kv_heads, "kv_heads", torch.int32, 1)
    if kv_heads.device != device:
        raise ValueError("kv_heads must be on the tensors' device")
    return kv_heads


def quantize_append_kv_heads(k_src: torch.Tensor, v_src: torch.Tensor, cache: "KVCache", kv_heads: torch.Tensor,
                             pos: int, bits: int = 4):
    """Quantize rows ``[pos, pos+T)`` of the KV heads ``kv_heads`` (int32, device) of a layer's
    ``k_src``/``v_src [B, Hkv, T, D]`` into a ``bits``-bit cache holding those heads
    (cache head i = layer head kv_heads[i])."""
    _req(k_src, "k_src", torch.float32, 4)
    _req(v_src, "v_src", torch.float32, 4)
    if k_src.shape != v_src.shape or k_src.device != v_src.device:
        raise ValueError("k_src and v_src must have one shape and device")
    B, Hkv, T, D = k_src.shape
    kv_heads = _heads_arg(kv_heads, k_src.device)
    Hs = kv_heads.numel()
    kc, ks, vc, vs = cache.tensors()
    for name, t, dt, nd in (("k_codes", kc, torch.uint8, 4), ("k_scales", ks, torch.float16, 3),
                            ("v_codes", vc, torch.uint8, 4), ("v_scales", vs, torch.float16, 3)):
        _req(t, name, dt, nd)
        if t.device != k_src.device:
            raise ValueError("all tensors must be on one device")
    if kc.shape[:2] != (B, Hs) or kc.shape[3] * 8 != D * bits or vc.shape != kc.shape or \
            ks.shape != kc.shape[:3] or vs.shape != ks.shape:
        raise ValueError("cache shape does not match src and kv_heads")
    _check(_lib.qkv_quantize_append_kv_heads(_ptr(k_src), _ptr(v_src), _ptr(kv_heads), Hs, _ptr(kc), _ptr(ks),
                                             _ptr(vc), _ptr(vs), B, Hkv, T, D, kc.shape[2], int(pos), int(bits),
                                             _stream(k_src)))


def decode_heads(q, cache: "KVCache", kv_heads: torch.Tensor, Hkv: int, kv_len, out, lse=None, softmax_scale=None,
                 num_splits=0, workspace=None, bits=4):
    """Decode for the query heads of the layer's KV heads ``kv_heads`` (int32, device) over a
    ``bits``-bit cache holding those heads; writes their rows of ``out`` (and ``lse``) only.
    ``q``/``out`` are the layer's ``[B, Hq, Sq, D]``; ``Hkv`` is the layer's KV head count."""
    _req(q, "q", torch.bfloat16, 4)
    B, Hq, Sq, D = q.shape
    kv_heads = _heads_arg(kv_heads, q.device)
    Hs = kv_heads.numel()
    if Hkv < 1 or Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    tensors = cache.tensors()
    kc, ks, vc, vs = tensors
    for name, t, dt, nd in (("k_codes", kc, torch.uint8, 4), ("k_scales", ks, torch.float16, 3),
                            ("v_codes", vc, torch.uint8, 4), ("v_scales", vs, torch.float16, 3)):
        _req(t, name, dt, nd)
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")
    if kc.shape[:2] != (B, Hs) or kc.shape[3] * 8 != D * bits or vc.shape != kc.shape or \
            ks.shape != kc.shape[:3] or vs.shape != ks.shape:
        raise ValueError("cache shape does not match q and kv_heads")
    out, lse = _outputs(q, out, lse, False)
    G = Hq // Hkv
    need = decode_workspace_bytes(B, G * Hs, Hs, Sq, kv_len, D, num_splits)
    if workspace is None and need > 0:
        workspace = _workspace(q.device, B * Hs, need)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.qkv_decode_heads(_ptr(q), _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs), _ptr(kv_heads), Hs, B, Hq, Hkv,
                                 Sq, int(kv_len), kc.shape[2], D, int(bits), _scale(softmax_scale, D),
                                 int(num_splits), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(q)))
    return out


def decode_mixed(q, parts, Hkv: int, kv_len, softmax_scale=None, num_splits=0, return_lse=False, out=None,
                 lse=None):
    """Decode of a layer whose KV heads are kept at different widths: ``parts`` is a list of
    ``(cache, kv_heads, bits)``, one per width, whose head lists cover the layer's ``Hkv`` KV
    heads once (one launch per part, all on the current stream)."""
    if sum(int(h.numel()) for _, h, _ in parts) != Hkv:
        raise ValueError("the parts' head lists must cover the layer's KV heads once")
    out, lse = _outputs(q, out, lse, return_lse)
    for cache, heads, bits in parts:
        decode_heads(q, cache, heads, Hkv, kv_len, out, lse, softmax_scale, num_splits, bits=bits)
    return (out, lse) if return_lse else out


def prefill_heads(q, cache: "KVCache", kv_heads: torch.Tensor, Hkv: int, kv_len, causal, out, lse=None,
                  softmax_scale=None, bits=4):
    """Prefill for the query heads of the layer's KV heads ``kv_heads`` (int32, device) over a
    ``bits``-bit cache holding those heads; writes their rows of ``out`` (and ``lse``) only.
    ``q``/``out`` are the layer's ``[B, Hq, Sq, D]``; ``Hkv`` is the layer's KV head count."""
    _req(q, "q", torch.bfloat16, 4)
    B, Hq, Sq, D = q.shape
    kv_heads = _heads_arg(kv_heads, q.device)
    Hs = kv_heads.numel()
    if Hkv < 1 or Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    kc, ks, vc, vs = cache.tensors()
    for name, t, dt, nd in (("k_codes", kc, torch.uint8, 4), ("k_scales", ks, torch.float16, 3),
                            ("v_codes", vc, torch.uint8, 4), ("v_scales", vs, torch.float16, 3)):
        _req(t, name, dt, nd)
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")
    if kc.shape[:2] != (B, Hs) or kc.shape[3] * 8 != D * bits or vc.shape != kc.shape or \
            ks.shape != kc.shape[:3] or vs.shape != ks.shape:
        raise ValueError("cache shape does not match q and kv_heads")
    out, lse = _outputs(q, out, lse, False)
    _check(_lib.qkv_prefill_heads(_ptr(q), _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs), _ptr(kv_heads), Hs, B, Hq, Hkv,
                                  Sq, int(kv_len), kc.shape[2], D, int(bits), _scale(softmax_scale, D),
                                  int(bool(causal)), _ptr(out), _ptr(lse), _stream(q)))
    return out


def prefill_mixed(q, parts, Hkv: int, kv_len, causal, softmax_scale=None, return_lse=False, out=None, lse=None):
    """Prefill of a layer whose KV heads are kept at different widths: ``parts`` is a list of
    ``(cache, kv_heads, bits)`` covering the layer's ``Hkv`` KV heads once (one launch per part)."""
    if sum(int(h.numel()) for _, h, _ in parts) != Hkv:
        raise ValueError("the parts' head lists must cover the layer's KV heads once")
    out, lse = _outputs(q, out, lse, return_lse)
    for cache, heads, bits in parts:
        prefill_heads(q, cache, heads, Hkv, kv_len, causal, out, lse, softmax_scale, bits=bits)
    return (out, lse) if return_lse else out


@dataclasses.dataclass
class AsymKVCache:
    """Caller-owned asymmetric group-wise int4 KV cache of one layer: unsigned
    nibble codes and one parameter word per group of ``group`` consecutive
    elements (fp16 scale in bits 0-15, zero point in bits 16-19)."""

    k_codes: torch.Tensor   # uint8 [B, Hkv, C, D/2]
    k_params: torch.Tensor  # int32 [B, Hkv, C, D/group]
    v_codes: torch.Tensor
    v_params: torch.Tensor
    group: int

    @staticmethod
    def empty(B: int, Hkv: int, C: int, D: int, group: int, device="cuda") -> "AsymKVCache":
        mk = lambda: torch.empty((B, Hkv, C, D // 2), dtype=torch.uint8, device=device)
        mp = lambda: torch.empty((B, Hkv, C, D // group), dtype=torch.int32, device=device)
        return AsymKVCache(mk(), mp(), mk(), mp(), int(group))

    def tensors(self):
        return self.k_codes, self.k_params, self.v_codes, self.v_params


def _asym_args(cache: AsymKVCache, device, B, Hkv, D):
    kc, kp, vc, vp = cache.tensors()
    for name, t, dt in (("k_codes", kc, torch.uint8), ("k_params", kp, torch.int32),
                        ("v_codes", vc, torch.uint8), ("v_params", vp, torch.int32)):
        _req(t, name, dt, 4)
        if t.device != device:
            raise ValueError("all tensors must be on one device")
    if kc.shape[:2] != (B, Hkv) or kc.shape[3] * 2 != D or vc.shape != kc.shape or \
            kp.shape != kc.shape[:3] + (D // max(cache.group, 1),) or vp.shape != kp.shape:
        raise ValueError("cache shape does not match")
    return kc, kp, vc, vp, kc.shape[2]


def quantize_append_kv_asym(k_src: torch.Tensor, v_src: torch.Tensor, cache: AsymKVCache, pos: int):
    """Quantize new K and V rows ``[B, Hkv, T, D]`` into rows ``[pos, pos+T)`` of an
    asymmetric group-wise cache (one launch)."""
    _req(k_src, "k_src", torch.float32, 4)
    _req(v_src, "v_src", torch.float32, 4)
    if k_src.shape != v_src.shape or k_src.device != v_src.device:
        raise ValueError("k_src and v_src must have one shape and device")
    B, Hkv, T, D = k_src.shape
    kc, kp, vc, vp, C = _asym_args(cache, k_src.device, B, Hkv, D)
    _check(_lib.qkv_quantize_append_kv_asym(_ptr(k_src), _ptr(v_src), _ptr(kc), _ptr(kp), _ptr(vc), _ptr(vp),
                                            B, Hkv, T, D, C, int(pos), int(cache.group), _stream(k_src)))


def decode_asym(q, cache: AsymKVCache, kv_len, softmax_scale=None, num_splits=0, return_lse=False, out=None,
                lse=None, workspace=None):
    """Decode attention of ``q [B, Hq, Sq, D]`` over rows ``[0, kv_len)`` of an asymmetric
    group-wise cache."""
    _req(q, "q", torch.bfloat16, 4)
    if not isinstance(cache, AsymKVCache):
        raise TypeError("cache must be an AsymKVCache")
    B, Hq, Sq, D = q.shape
    Hkv = int(cache.k_codes.shape[1]) if cache.k_codes.dim() == 4 else 0
    kc, kp, vc, vp, C = _asym_args(cache, q.device, B, Hkv, D)
    out, lse = _outputs(q, out, lse, return_lse)
    need = decode_workspace_bytes(B, Hq, Hkv, Sq, kv_len, D, num_splits)
    if workspace is None and need > 0:
        workspace = _workspace(q.device, B * Hkv, need)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.qkv_decode_asym(_ptr(q), _ptr(kc), _ptr(kp), _ptr(vc), _ptr(vp), B, Hq, Hkv, Sq, int(kv_len),
                                C, D, int(cache.group), _scale(softmax_scale, D), int(num_splits), _ptr(out),
                                _ptr(lse), _ptr(workspace), ws_bytes, _stream(q)))
    return (out, lse) if return_lse else out


def prefill_asym(q, cache: AsymKVCache, kv_len, causal, softmax_scale=None, return_lse=False, out=None,
                 lse=None):
    """Prefill attention of ``q [B, Hq, Sq, D]`` over rows ``[0, kv_len)`` of an
    asymmetric group-wise cache (causal: bottom-right aligned, as ``prefill``)."""
    _req(q, "q", torch.bfloat16, 4)
    if not isinstance(cache, AsymKVCache):
        raise TypeError("cache must be an AsymKVCache")
    B, Hq, Sq, D = q.shape
    Hkv = int(cache.k_codes.shape[1]) if cache.k_codes.dim() == 4 else 0
    kc, kp, vc, vp, C = _asym_args(cache, q.device, B, Hkv, D)
    out, lse = _outputs(q, out, lse, return_lse)
    _check(_lib.qkv_prefill_asym(_ptr(q), _ptr(kc), _ptr(kp), _ptr(vc), _ptr(vp), B, Hq, Hkv, Sq, int(kv_len),
                                 C, D, int(cache.group), _scale(softmax_scale, D), int(bool(causal)), _ptr(out),
                                 _ptr(lse), _stream(q)))
    return (out, lse) if return_lse else out


def decode_append(q, k_new, v_new, cache, pos, softmax_scale=None, num_splits=0, return_lse=False,
                  out=None, lse=None, workspace=None):
    """One decode step in one launch: quantize ``k_new``/``v_new [B, Hkv, n_new, D]``
    into cache rows ``[pos, pos+n_new)``, then decode ``q`` over rows ``[0, pos+n_new)``.
    Same results as ``quantize_append_kv`` followed by ``decode``."""
    tensors = cache.tensors() if isinstance(cache, KVCache) else tuple(cache)
    _req(k_new, "k_new", torch.float32, 4)
    _req(v_new, "v_new", torch.float32, 4)
    if k_new.shape != v_new.shape or k_new.device != q.device or v_new.device != q.device:
        raise ValueError("k_new and v_new must have one shape and q's device")
    n_new = k_new.shape[2]
    B, Hq, Hkv, Sq, kv_len, C, D = _attn_args(q, tensors, int(pos) + n_new)
    if k_new.shape != (B, Hkv, n_new, D):
        raise ValueError("k_new shape does not match the cache")
    out, lse = _outputs(q, out, lse, return_lse)
    need = decode_workspace_bytes(B, Hq, Hkv, Sq, kv_len, D, num_splits)
    if workspace is None and need > 0:
        workspace = _workspace(q.device, B * Hkv, need)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    kc, ks, vc, vs = tensors
    _check(_lib.qkv_decode_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs),
                                  B, Hq, Hkv, Sq, int(pos), n_new, C, D, _scale(softmax_scale, D),
                                  int(num_splits), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                  _stream(q)))
    return (out, lse) if return_lse else out


def decode_paged(q, cache, kv_lens=None, block_table=None, k_new=None, v_new=None, max_kv_len=None,
                 softmax_scale=None, num_splits=0, return_lse=False, out=None, lse=None, workspace=None):
    """Decode step over a ragged, optionally paged cache, in one launch.

    Sequence ``b`` first gets its new rows ``k_new``/``v_new [B, Hkv, n_new, D]``
    (optional, fp32) quantized into its rows ``[kv_lens[b], kv_lens[b]+n_new)``,
    then ``q[b]`` attends its rows ``[0, kv_lens[b]+n_new)``.

    * ``cache``: a :class:`KVCache` whose tensors are a page pool
      ``[num_pages, Hkv, page_size, D/2]`` / ``[num_pages, Hkv, page_size]``.
      Without ``block_table`` it is an ordinary cache ``[B', Hkv, C, ...]``,
      ``B' >= B``, and sequence ``b`` uses entry ``b``.
    * ``kv_lens``: int32 ``[B]`` device tensor of rows already cached (None:
      every sequence holds ``max_kv_len - n_new``).
    * ``block_table``: int32 ``[B, max_pages]`` device tensor of page ids
      (``page_size`` a multiple of 32), or None.
    * ``max_kv_len``: upper bound of ``kv_lens[b] + n_new``; the split plan and
      the workspace follow it (default: the capacity ``max_pages * page_size``;
      a tight bound avoids splits that find nothing to do).
    """
    tensors = cache.tensors() if isinstance(cache, KVCache) else tuple(cache)
    _req(q, "q", torch.bfloat16, 4)
    kc, ks, vc, vs = tensors
    for name, t, dt, nd in (("k_codes", kc, torch.uint8, 4), ("k_scales", ks, torch.float16, 3),
                            ("v_codes", vc, torch.uint8, 4), ("v_scales", vs, torch.float16, 3)):
        _req(t, name, dt, nd)
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")
    B, Hq, Sq, D = q.shape
    num_pages, Hkv, page_size, half = kc.shape
    if half * 2 != D or vc.shape != kc.shape or ks.shape != kc.shape[:3] or vs.shape != ks.shape:
        raise ValueError("cache shape does not match q")
    if block_table is not None:
        _req(block_table, "block_table", torch.int32, 2)
        if block_table.shape[0] != B or block_table.device != q.device:
            raise ValueError("block_table must be [B, max_pages] on q's device")
        max_pages = block_table.shape[1]
    else:
        max_pages = 1
    if kv_lens is not None:
        _req(kv_lens, "kv_lens", torch.int32, 1)
        if kv_lens.shape[0] != B or kv_lens.device != q.device:
            raise ValueError("kv_lens must be [B] on q's device")
    n_new = 0
    if k_new is not None or v_new is not None:
        if k_new is None or v_new is None:
            raise ValueError("pass both k_new and v_new, or neither")
        _req(k_new, "k_new", torch.float32, 4)
        _req(v_new, "v_new", torch.float32, 4)
        n_new = k_new.shape[2]
        if k_new.shape != (B, Hkv, n_new, D) or v_new.shape != k_new.shape or \
                k_new.device != q.device or v_new.device != q.device:
            raise ValueError("k_new and v_new must be [B, Hkv, n_new, D] on q's device")
    if max_kv_len is None:
        max_kv_len = max_pages * page_size
    max_kv_len = int(max_kv_len)
    out, lse = _outputs(q, out, lse, return_lse)
    need = decode_workspace_bytes(B, Hq, Hkv, Sq, max_kv_len, D, num_splits)
    if workspace is None and need > 0:
        workspace = _workspace(q.device, B * Hkv, need)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.qkv_decode_paged(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs),
                                 _ptr(block_table), _ptr(kv_lens), B, Hq, Hkv, Sq, n_new, max_kv_len,
                                 page_size, max_pages, num_pages, D, _scale(softmax_scale, D),
                                 int(num_splits), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                 _stream(q)))
    return (out, lse) if return_lse else out


@dataclasses.dataclass
class DecodeBuffer:
    """INT8 decode buffer of one layer: the newest tokens of every (batch, KV
    head) as INT8 codes under one universal scale each (TurboAttention §3.3).

    ``length`` is the number of buffered rows (host-side, the same for every
    sequence); :func:`decode_buffered` advances it, :func:`buffer_flush`
    resets it.
    """

    k: torch.Tensor      # int8 [B, Hkv, rows, D]
    v: torch.Tensor
    k_s8: torch.Tensor   # float32 [B, Hkv]
    v_s8: torch.Tensor
    length: int = 0

    @staticmethod
    def empty(B: int, Hkv: int, D: int, rows: int = 64, device="cuda") -> "DecodeBuffer":
        mk = lambda: torch.zeros((B, Hkv, rows, D), dtype=torch.int8, device=device)
        ms = lambda: torch.zeros((B, Hkv), dtype=torch.float32, device=device)
        return DecodeBuffer(mk(), mk(), ms(), ms(), 0)

    @property
    def rows(self) -> int:
        return self.k.shape[2]

    def _check(self, device):
        for name, t, dt, nd in (("k", self.k, torch.int8, 4), ("v", self.v, torch.int8, 4),
                                ("k_s8", self.k_s8, torch.float32, 2), ("v_s8", self.v_s8, torch.float32, 2)):
            _req(t, f"buffer.{name}", dt, nd)
            if t.device != device:
                raise ValueError("all tensors must be on one device")
        if self.v.shape != self.k.shape or self.k_s8.shape != self.k.shape[:2] or self.v_s8.shape != self.k_s8.shape:
            raise ValueError("inconsistent buffer shapes")


def buffer_scale(cache, kv_len: int, buf: "DecodeBuffer"):
    """Set ``buf``'s universal scales from cache rows ``[0, kv_len)``:
    ``s8 = 7 * max_t scale[t] / 127`` per (batch, KV head), K and V."""
    kc, ks, vc, vs = cache.tensors() if isinstance(cache, KVCache) else tuple(cache)
    _req(ks, "k_scales", torch.float16, 3)
    _req(vs, "v_scales", torch.float16, 3)
    buf._check(ks.device)
    B, Hkv, C = ks.shape
    if vs.shape != ks.shape or buf.k_s8.shape != (B, Hkv):
        raise ValueError("cache and buffer shapes do not match")
    _check(_lib.qkv_buffer_scale(_ptr(ks), _ptr(vs), B, Hkv, int(kv_len), C, _ptr(buf.k_s8), _ptr(buf.v_s8),
                                 _stream(ks)))


def buffer_flush(buf: "DecodeBuffer", cache, pos: int):
    """Quantize the buffered rows into int4 cache rows ``[pos, pos + buf.length)``
    and empty the buffer (its scales are kept)."""
    kc, ks, vc, vs = cache.tensors() if isinstance(cache, KVCache) else tuple(cache)
    for name, t, dt, nd in (("k_codes", kc, torch.uint8, 4), ("k_scales", ks, torch.float16, 3),
                            ("v_codes", vc, torch.uint8, 4), ("v_scales", vs, torch.float16, 3)):
        _req(t, name, dt, nd)
    buf._check(kc.device)
    B, Hkv, C, half = kc.shape
    D = buf.k.shape[3]
    if buf.k.shape[:2] != (B, Hkv) or half * 2 != D or vc.shape != kc.shape or ks.shape != (B, Hkv, C) \
            or vs.shape != ks.shape:
        raise ValueError("cache and buffer shapes do not match")
    _check(_lib.qkv_buffer_flush(_ptr(buf.k), _ptr(buf.v), _ptr(buf.k_s8), _ptr(buf.v_s8), buf.rows, buf.length,
                                 _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs), B, Hkv, D, C, int(pos), _stream(kc)))
    buf.length = 0


def decode_buffered_workspace_bytes(B, Hq, Hkv, Sq, kv_len, D, num_splits=0) -> int:
    return int(_lib.qkv_decode_buffered_workspace_bytes(B, Hq, Hkv, Sq, kv_len, D, num_splits))


def decode_buffered(q, cache, kv_len, buf: "DecodeBuffer", k_new=None, v_new=None, softmax_scale=None,
                    num_splits=0, return_lse=False, out=None, lse=None, workspace=None):
    """Decode step over int4 cache rows ``[0, kv_len)`` followed by the buffered
    INT8 rows, in one launch.  New rows ``k_new``/``v_new [B, Hkv, n, D]``
    (optional, fp32) are first quantized into the buffer under its universal
    scales (outliers clamped) and attended; ``buf.length`` grows by ``n``."""
    tensors = cache.tensors() if isinstance(cache, KVCache) else tuple(cache)
    B, Hq, Hkv, Sq, _, C, D = _attn_args(q, tensors, kv_len)
    buf._check(q.device)
    if buf.k.shape[:2] != (B, Hkv) or buf.k.shape[3] != D:
        raise ValueError("buffer shape does not match the cache")
    n_new = 0
    if k_new is not None or v_new is not None:
        if k_new is None or v_new is None:
            raise ValueError("pass both k_new and v_new, or neither")
        _req(k_new, "k_new", torch.float32, 4)
        _req(v_new, "v_new", torch.float32, 4)
        n_new = k_new.shape[2]
        if k_new.shape != (B, Hkv, n_new, D) or v_new.shape != k_new.shape or \
                k_new.device != q.device or v_new.device != q.device:
            raise ValueError("k_new and v_new must be [B, Hkv, n_new, D] on q's device")
    out, lse = _outputs(q, out, lse, return_lse)
    need = decode_buffered_workspace_bytes(B, Hq, Hkv, Sq, int(kv_len), D, num_splits)
    if workspace is None and need > 0:
        workspace = _workspace(q.device, B * Hkv, need)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    kc, ks, vc, vs = tensors
    _check(_lib.qkv_decode_buffered(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs),
                                    _ptr(buf.k), _ptr(buf.v), _ptr(buf.k_s8), _ptr(buf.v_s8), B, Hq, Hkv, Sq,
                                    int(kv_len), C, buf.rows, buf.length, n_new, D, _scale(softmax_scale, D),
                                    int(num_splits), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(q)))
    buf.length += n_new
    return (out, lse) if return_lse else out


def prefill(q, cache, kv_len, causal, softmax_scale=None, return_lse=False, out=None, lse=None, bits=4):
    """Prefill attention of ``q [B, Hq, Sq, D]`` over cache rows ``[0, kv_len)``;
    ``bits`` = 2, 3 or 4 is the width of the cache's codes."""
    tensors = cache.tensors() if isinstance(cache, KVCache) else tuple(cache)
    B, Hq, Hkv, Sq, kv_len, C, D = _attn_args(q, tensors, kv_len, bits)
    out, lse = _outputs(q, out, lse, return_lse)
    kc, ks, vc, vs = tensors
    if bits == 4:
        _check(_lib.qkv_prefill(_ptr(q), _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs), B, Hq, Hkv, Sq, kv_len,
                                C, D, _scale(softmax_scale, D), int(bool(causal)), _ptr(out), _ptr(lse),
                                _stream(q)))
    else:
        _check(_lib.qkv_prefill_bits(_ptr(q), _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs), B, Hq, Hkv, Sq, kv_len,
                                     C, D, int(bits), _scale(softmax_scale, D), int(bool(causal)), _ptr(out),
                                     _ptr(lse), _stream(q)))
    return (out, lse) if return_lse else out

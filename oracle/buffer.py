"""INT8 decode-buffer oracle (TEST INFRASTRUCTURE ONLY; see the package docstring).

Follows TurboAttention (arXiv 2412.08585):

* §3.3 (decoding buffer): the newest tokens of a sequence -- at most n_b of
  them, n_b = 64 -- are kept in a buffer with 8-bit symmetric quantization
  under one universal scale; values outside that scale's range are clamped,
  so rows already in the buffer are never re-quantized.  When the buffer is
  full its rows are compressed further to the low-bit cache format.
* Appendix/implementation paragraph of §5: only new tokens are quantized to
  INT8; the universal scale is the previous cache's value-range maximum, and
  newer tokens beyond it are clamped.
* §2.3 (progressive quantization): compressing INT8 rows to lower bit widths
  goes through their dequantized values.

The displayed equations of those sections are lost in the page text, so the
following readings are used (each plain and consistent with the prose):

* universal scale s8 per (batch, KV head), fp32: the cache's value-range
  maximum over its rows ``[0, L)`` is ``7 * max_t s4[t]`` (the int4 row scale
  is absmax / 7, so 7 * s4 recovers each row's absmax up to the fp16 rounding
  of s4; exact in fp32), and ``s8 = that / 127`` with IEEE fp32 division;
  an empty or all-zero cache gives ``s8 = 0``;
* INT8 code: ``clamp(rint(x / s8), -127, 127)`` with IEEE fp32 division and
  round-half-to-even (symmetric 8-bit, the same rounding as the int4 codes);
  ``s8 = 0`` gives code 0;
* dequantized value: ``s8 * code`` (exact in fp64);
* flush (INT8 -> int4): each buffered row is dequantized as the fp32 product
  ``fp32(s8 * code)`` and quantized with the int4 row quantizer;
* decode over the buffered cache: plain attention over the rows
  ``[0, L)`` of the int4 cache followed by the ``T`` buffered rows.
"""
from __future__ import annotations

import numpy as np

from .attention import bf16_bits_to_f64, _attend
from .quantize import dequantize_cache, quantize_rows

__all__ = ["buffer_scale", "quantize_int8", "dequantize_int8", "flush_rows", "attention_buffered"]

_SEVEN = np.float32(7.0)
_I8MAX = np.float32(127.0)


def buffer_scale(scale_bits: np.ndarray, L: int) -> np.ndarray:
    """Universal INT8 scale from int4 row scales ``[..., C]`` (fp16 bits), rows ``[0, L)``.

    Returns fp32 ``[...]``: ``(7 * max_t s4[t]) / 127``; 0 when ``L == 0``.
    """
    s = np.asarray(scale_bits, dtype=np.uint16)[..., :L].view(np.float16).astype(np.float32)
    if L == 0:
        return np.zeros(s.shape[:-1], np.float32)
    amax = s.max(axis=-1) * _SEVEN          # exact: an 11-bit significand times 7
    return (amax / _I8MAX).astype(np.float32)


def quantize_int8(x: np.ndarray, s8: np.ndarray) -> np.ndarray:
    """INT8 codes of fp32 rows ``x [..., D]`` under per-row-group scales ``s8 [...]``."""
    x = np.asarray(x, dtype=np.float32)
    s = np.asarray(s8, dtype=np.float32)[..., None]
    zero = s == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        r = x / np.where(zero, np.float32(1.0), s)      # fp32 IEEE division
    c = np.clip(np.rint(r), -127, 127)                  # round half to even, clamp outliers
    return np.where(zero, 0, c).astype(np.int8)


def dequantize_int8(codes: np.ndarray, s8: np.ndarray) -> np.ndarray:
    """Exact fp64 values ``s8 * code``."""
    return np.asarray(codes, dtype=np.int8).astype(np.float64) * \
        np.asarray(s8, dtype=np.float32).astype(np.float64)[..., None]


def flush_rows(codes: np.ndarray, s8: np.ndarray):
    """int4 ``(codes, scale_bits)`` of buffered INT8 rows ``[..., T, D]`` (scales ``[...]``)."""
    c = np.asarray(codes, dtype=np.int8).astype(np.float32)
    x = c * np.asarray(s8, dtype=np.float32)[..., None, None]    # fp32 product, rounded once
    return quantize_rows(x.astype(np.float32))


def attention_buffered(q_bits, k_codes, k_scales, v_codes, v_scales, L, k_tail, v_tail, k_s8, v_s8, T,
                       softmax_scale):
    """Attention of ``q`` over int4 rows ``[0, L)`` then buffered INT8 rows ``[0, T)``.

    ``k_tail``/``v_tail`` int8 ``[B, Hkv, >=T, D]``, ``k_s8``/``v_s8`` fp32 ``[B, Hkv]``.
    Returns fp64 ``(out [B, Hq, Sq, D], lse [B, Hq, Sq])``.
    """
    B, Hq, Sq, D = q_bits.shape
    Hkv = k_codes.shape[1]
    G = Hq // Hkv
    scale = float(np.float32(softmax_scale))
    out = np.empty((B, Hq, Sq, D))
    lse = np.empty((B, Hq, Sq))
    for b in range(B):
        for g in range(Hkv):
            kd = np.concatenate([dequantize_cache(k_codes[b:b + 1, g:g + 1], k_scales[b:b + 1, g:g + 1], L)[0, 0],
                                 dequantize_int8(k_tail[b, g, :T], k_s8[b, g])], axis=0)
            vd = np.concatenate([dequantize_cache(v_codes[b:b + 1, g:g + 1], v_scales[b:b + 1, g:g + 1], L)[0, 0],
                                 dequantize_int8(v_tail[b, g, :T], v_s8[b, g])], axis=0)
            for h in range(g * G, (g + 1) * G):
                qd = bf16_bits_to_f64(q_bits[b, h])
                out[b, h], lse[b, h] = _attend(qd, kd, vd, scale, False, 0, 512)
    return out, lse

"""int4 KV quantizer oracle (TEST INFRASTRUCTURE ONLY; see the package docstring).

Follows:

* "Quantized Cross-Attention: Extending FlashAttention-3 with In-SRAM
  Dequantization", §4.1 (kernel signature): the KV cache is stored as packed
  low-bit codes ``[batch, heads, seq_kv, dim*bits/32]`` words plus scales
  ``[batch, heads, seq_kv, dim/GROUP_SIZE]``; here bits = 4 and GROUP_SIZE =
  dim, i.e. one scale per (token, KV head).
* Same page, §3.1 (the inline dequant fragment): a code is taken from a packed
  word with ``& 0xF``, i.e. the first value sits in the low nibble.
* "Attention Quantization" topic listing, Open-TQ-Metal abstract: the KV cache
  is quantized to int4 on the fly as tokens are produced.
* TurboAttention (arXiv 2412.08585) §2.1: each decode step appends the new
  token's k/v to the cache (K_t = K_{t-1} | k_t).

The pages give no formula for the scale; the reading used (absmax / 7 in
fp32, rounded to fp16, codes by IEEE fp32 division by the rounded scale, then
round-half-even and clamp to [-8, 7]) is the one the library is specified
with.  Everything here runs in fp32 (the precision that specification fixes),
then dequantization is exact in fp64.
"""
from __future__ import annotations

import numpy as np

__all__ = ["quantize_rows", "dequantize_rows", "quantize_append", "dequantize_cache"]

_SEVEN = np.float32(7.0)


def quantize_rows(x: np.ndarray):
    """Quantize rows of ``x`` (fp32, last axis = head dim D, D even).

    Returns ``(codes, scale_bits)``: ``codes`` uint8 ``[..., D/2]`` where byte
    ``i`` holds element ``2i`` in bits 0-3 and element ``2i+1`` in bits 4-7,
    each as a two's-complement 4-bit value; ``scale_bits`` uint16 ``[...]``,
    the fp16 bit pattern of the row's scale.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.shape[-1] % 2:
        raise ValueError("head dim must be even")
    amax = np.max(np.abs(x), axis=-1)                  # exact in fp32
    s16 = (amax / _SEVEN).astype(np.float16)           # fp32 IEEE divide, then RNE to fp16
    s = s16.astype(np.float32)[..., None]              # exact widening
    zero = s == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        r = x / np.where(zero, np.float32(1.0), s)     # fp32 IEEE divide by the rounded scale
    c = np.clip(np.rint(r), -8, 7)                     # rint = round half to even
    c = np.where(zero, 0, c).astype(np.int8)
    nib = c.view(np.uint8) & np.uint8(0x0F)
    codes = nib[..., 0::2] | (nib[..., 1::2] << np.uint8(4))
    return np.ascontiguousarray(codes, dtype=np.uint8), s16.view(np.uint16)


def _unpack(codes: np.ndarray) -> np.ndarray:
    """uint8 ``[..., D/2]`` -> int8 codes ``[..., D]`` (low nibble = even element)."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = (codes & np.uint8(0x0F)).astype(np.int16)
    hi = (codes >> np.uint8(4)).astype(np.int16)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.int16)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    out = np.where(out >= 8, out - 16, out)            # two's complement nibble
    return out.astype(np.int8)


def dequantize_rows(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Exact fp64 values ``scale * code`` of quantized rows."""
    c = _unpack(codes).astype(np.float64)
    s = np.asarray(scale_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    return c * s[..., None]


def quantize_append(src: np.ndarray, codes: np.ndarray, scales: np.ndarray, pos: int):
    """Quantize ``src`` fp32 ``[B, Hkv, T, D]`` into cache rows ``[pos, pos+T)``.

    ``codes`` uint8 ``[B, Hkv, C, D/2]`` and ``scales`` uint16 ``[B, Hkv, C]``
    are updated in place (rows outside ``[pos, pos+T)`` are left untouched);
    they are also returned.
    """
    T = src.shape[2]
    C = codes.shape[2]
    if pos < 0 or pos + T > C:
        raise ValueError("append range outside the cache")
    qc, qs = quantize_rows(src)
    codes[:, :, pos:pos + T, :] = qc
    scales[:, :, pos:pos + T] = qs
    return codes, scales


def dequantize_cache(codes: np.ndarray, scales: np.ndarray, n: int | None = None) -> np.ndarray:
    """fp64 ``[B, Hkv, n, D]`` of the first ``n`` cached rows (all rows if None)."""
    if n is None:
        n = codes.shape[2]
    return dequantize_rows(codes[:, :, :n, :], scales[:, :, :n])

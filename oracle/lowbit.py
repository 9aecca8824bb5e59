"""2- and 3-bit KV row quantizer oracle (TEST INFRASTRUCTURE ONLY; see the package docstring).

Follows "Quantized Cross-Attention: Extending FlashAttention-3 with In-SRAM
Dequantization": §4.1's kernel takes the bit width as a parameter (codes
``[.., seq_kv, dim*bits/32]`` words, scales ``[.., seq_kv, dim/GROUP_SIZE]``)
and §3.3 and its throughput tables treat 2- and 3-bit codes beside 4-bit
ones.  TurboAttention (arXiv 2412.08585) §3.2 keeps some heads at 2 bits.

Readings (the pages give no formula for these widths):

* the int4 rule widened to b bits: scale = fp16(absmax / qmax) with
  qmax = 2^(b-1) - 1 (IEEE fp32 division, one rounding to fp16; 7, 3 and 1
  for b = 4, 3, 2), code = clamp(rint(x / scale), -2^(b-1), qmax) by IEEE
  fp32 division with round-half-to-even; a zero scale gives zero codes;
* 2-bit rows: four codes per byte, element i in bits 2(i mod 4) .. +1 of
  byte i // 4, two's complement (D/4 bytes per row);
* 3-bit rows: the low two bits of every code packed as a 2-bit row (D/4
  bytes), followed by the top (sign) bit of every code, element i in bit
  i mod 8 of byte D/4 + i // 8 (3D/8 bytes per row).  The page's own 3-bit
  layout (ten codes per 32-bit word) is garbled in the text (it names eleven
  lanes for ten codes); two planes keep every load of a row aligned;
* dequantized value: scale * code, exact in fp64.
"""
from __future__ import annotations

import numpy as np

__all__ = ["row_bytes", "quantize_rows_bits", "unpack_bits", "dequantize_rows_bits", "dequantize_cache_bits",
           "attention_bits"]


def row_bytes(D: int, bits: int) -> int:
    """Bytes of one packed row of D codes."""
    if bits not in (2, 3, 4):
        raise ValueError("bits must be 2, 3 or 4")
    return D * bits // 8


def _codes(x: np.ndarray, bits: int):
    x = np.ascontiguousarray(x, dtype=np.float32)
    qmax = np.float32(2 ** (bits - 1) - 1)
    amax = np.max(np.abs(x), axis=-1)
    s16 = (amax / qmax).astype(np.float16)               # fp32 IEEE divide, then RNE to fp16
    s = s16.astype(np.float32)[..., None]
    zero = s == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        r = x / np.where(zero, np.float32(1.0), s)       # fp32 IEEE divide by the rounded scale
    c = np.clip(np.rint(r), -(2 ** (bits - 1)), 2 ** (bits - 1) - 1)
    return np.where(zero, 0, c).astype(np.int8), s16.view(np.uint16)


def _pack2(u: np.ndarray) -> np.ndarray:
    """Unsigned 2-bit fields [..., D] -> bytes [..., D/4], element i at bits 2(i % 4)."""
    u = u.astype(np.uint8)
    return (u[..., 0::4] | (u[..., 1::4] << 2) | (u[..., 2::4] << 4) | (u[..., 3::4] << 6)).astype(np.uint8)


def _pack1(u: np.ndarray) -> np.ndarray:
    """Bits [..., D] -> bytes [..., D/8], element i at bit i % 8."""
    u = u.astype(np.uint8)
    out = np.zeros(u.shape[:-1] + (u.shape[-1] // 8,), np.uint8)
    for k in range(8):
        out |= u[..., k::8] << k
    return out


def quantize_rows_bits(x: np.ndarray, bits: int):
    """Quantize fp32 rows ``x [..., D]`` to ``bits``-bit codes.

    Returns ``(codes, scale_bits)``: packed uint8 ``[..., row_bytes(D, bits)]``
    and the fp16 bit pattern of each row's scale.
    """
    D = np.shape(x)[-1]
    if D % 8:
        raise ValueError("head dim must be a multiple of 8")
    c, s = _codes(x, bits)
    u = c.view(np.uint8)
    if bits == 4:
        nib = u & np.uint8(0x0F)
        packed = nib[..., 0::2] | (nib[..., 1::2] << np.uint8(4))
    elif bits == 2:
        packed = _pack2(u & np.uint8(3))
    elif bits == 3:
        packed = np.concatenate([_pack2(u & np.uint8(3)), _pack1((u >> np.uint8(2)) & np.uint8(1))], axis=-1)
    else:
        raise ValueError("bits must be 2, 3 or 4")
    return np.ascontiguousarray(packed, dtype=np.uint8), s


def unpack_bits(codes: np.ndarray, D: int, bits: int) -> np.ndarray:
    """Packed rows ``[..., row_bytes]`` -> signed codes int8 ``[..., D]``."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (D,), np.int16)
    if bits == 4:
        out[..., 0::2] = codes & 0x0F
        out[..., 1::2] = codes >> 4
        return np.where(out >= 8, out - 16, out).astype(np.int8)
    lo = codes[..., : D // 4]
    for k in range(4):
        out[..., k::4] = (lo >> (2 * k)) & 3
    if bits == 2:
        return np.where(out >= 2, out - 4, out).astype(np.int8)
    if bits == 3:
        hi = codes[..., D // 4: D // 4 + D // 8]
        for k in range(8):
            out[..., k::8] |= ((hi >> k) & 1).astype(np.int16) << 2
        return np.where(out >= 4, out - 8, out).astype(np.int8)
    raise ValueError("bits must be 2, 3 or 4")


def dequantize_rows_bits(codes: np.ndarray, scale_bits: np.ndarray, D: int, bits: int) -> np.ndarray:
    """Exact fp64 values ``scale * code`` of packed rows."""
    c = unpack_bits(codes, D, bits).astype(np.float64)
    s = np.asarray(scale_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    return c * s[..., None]


def dequantize_cache_bits(codes: np.ndarray, scales: np.ndarray, D: int, bits: int, n: int | None = None):
    """fp64 ``[B, Hkv, n, D]`` of the first ``n`` cached rows (all rows if None)."""
    if n is None:
        n = codes.shape[2]
    return dequantize_rows_bits(codes[:, :, :n, :], scales[:, :, :n], D, bits)


def attention_bits(q_bits, k_codes, k_scales, v_codes, v_scales, kv_len, softmax_scale, bits, causal=False):
    """``attention`` (same definition, fp64) over a cache of ``bits``-bit rows.

    ``k_codes``/``v_codes`` uint8 ``[B, Hkv, C, row_bytes(D, bits)]``.
    """
    from .attention import _attend, bf16_bits_to_f64
    B, Hq, Sq, D = q_bits.shape
    Hkv = k_codes.shape[1]
    G = Hq // Hkv
    scale = float(np.float32(softmax_scale))
    out = np.empty((B, Hq, Sq, D))
    lse = np.empty((B, Hq, Sq))
    for b in range(B):
        for g in range(Hkv):
            kd = dequantize_cache_bits(k_codes[b:b + 1, g:g + 1], k_scales[b:b + 1, g:g + 1], D, bits, kv_len)[0, 0]
            vd = dequantize_cache_bits(v_codes[b:b + 1, g:g + 1], v_scales[b:b + 1, g:g + 1], D, bits, kv_len)[0, 0]
            for h in range(g * G, (g + 1) * G):
                out[b, h], lse[b, h] = _attend(bf16_bits_to_f64(q_bits[b, h]), kd, vd, scale, causal, kv_len - Sq, 512)
    return out, lse

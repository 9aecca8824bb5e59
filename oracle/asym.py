"""Asymmetric group-wise int4 KV row quantizer oracle (TEST INFRASTRUCTURE ONLY; see the package docstring).

Follows TurboAttention (arXiv 2412.08585) §2.3 (progressive quantization:
asymmetric INT4 with a scale s and a zero point z, dequantized value
s (code - z); its equations are lost in the text, the prose names s and z) and
§3.1 (block-wise progressive quantization keeps asymmetric INT4 groups), and
"Quantized Cross-Attention" §4.1 (scales ``[.., seq_kv, dim/GROUP_SIZE]``: one
scale per group of GROUP_SIZE consecutive elements of a row).

Readings (no page gives the formulas):

* groups: ``g`` consecutive elements of one row (one token of one KV head),
  ``g`` dividing the head dim; each group has its own scale and zero point;
* the group's range includes zero: lo = min(0, min x), hi = max(0, max x), so
  0 is exactly representable and the zero point lies in [0, 15];
* scale s = fp16(fp32(hi - lo) / 15): IEEE fp32 subtraction and division, one
  rounding to fp16 (round to nearest even);
* zero point z = clamp(rint(-lo / s), 0, 15) by IEEE fp32 division by the
  rounded scale, round half to even;
* code u = clamp(rint(x / s) + z, 0, 15), unsigned 4 bits, element 2i in the
  low nibble of byte i (as the int4 rows);
* a zero scale (an all-zero group) gives z = 0 and all codes 0;
* dequantized value: s (u - z), exact in fp64.

Storage: codes uint8 ``[..., D/2]``, scales fp16 bits ``[..., D/g]``, zero
points uint8 ``[..., D/g]``.  ``quantize_rows_asym`` packs codes in element
order (element 2i in the low nibble of byte i).  The cache stores the same
nibbles in a fixed order inside each row, one for K rows and one for V rows
(``cache_order``), so that each matrix-product block of the kernels reads
elements of one group only; the order is a layout choice, not part of the
quantization:

* K rows, chunk c = 4 k + j (elements 8c .. 8c+7, k < D/32, j < 4) is stored
  as dword (D/32) j + k, its element i in nibble i;
* V rows, element e = 16 p + w (p < D/16, w < 16) is stored, for D = 128,
  in nibble p of dword w; for D = 64 in nibble p + 4 (w // 8) of dword w % 8.
"""
from __future__ import annotations

import numpy as np

__all__ = ["quantize_rows_asym", "unpack_asym", "dequantize_rows_asym", "dequantize_cache_asym", "attention_asym",
           "cache_order", "to_cache_order", "from_cache_order"]


def _check(D: int, group: int):
    if group < 2 or D % group or group % 2:
        raise ValueError("group must be even and divide the head dim")


def quantize_rows_asym(x: np.ndarray, group: int):
    """Quantize fp32 rows ``x [..., D]`` in groups of ``group`` elements.

    Returns ``(codes, scale_bits, zeros)``: packed uint8 ``[..., D/2]``, the fp16
    bit pattern of each group's scale ``[..., D/group]`` and its zero point
    (uint8) ``[..., D/group]``.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    D = x.shape[-1]
    _check(D, group)
    xg = x.reshape(x.shape[:-1] + (D // group, group))
    lo = np.minimum(np.min(xg, axis=-1), np.float32(0.0))
    hi = np.maximum(np.max(xg, axis=-1), np.float32(0.0))
    s16 = ((hi - lo) / np.float32(15.0)).astype(np.float16)       # fp32 sub and divide, RNE to fp16
    s = s16.astype(np.float32)
    zero = s == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        sd = np.where(zero, np.float32(1.0), s)
        z = np.clip(np.rint(-lo / sd), 0, 15)                    # fp32 divide by the rounded scale
        u = np.clip(np.rint(xg / sd[..., None]) + z[..., None], 0, 15)
    z = np.where(zero, 0, z).astype(np.uint8)
    u = np.where(zero[..., None], 0, u).astype(np.uint8).reshape(x.shape)
    codes = (u[..., 0::2] | (u[..., 1::2] << np.uint8(4))).astype(np.uint8)
    return np.ascontiguousarray(codes), s16.view(np.uint16), z


def unpack_asym(codes: np.ndarray) -> np.ndarray:
    """Packed rows ``[..., D/2]`` -> unsigned codes uint8 ``[..., D]``."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (2 * codes.shape[-1],), np.uint8)
    out[..., 0::2] = codes & 0x0F
    out[..., 1::2] = codes >> 4
    return out


def dequantize_rows_asym(codes: np.ndarray, scale_bits: np.ndarray, zeros: np.ndarray, group: int) -> np.ndarray:
    """Exact fp64 values ``s (u - z)`` of packed rows."""
    u = unpack_asym(codes).astype(np.float64)
    D = u.shape[-1]
    _check(D, group)
    s = np.asarray(scale_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    z = np.asarray(zeros, dtype=np.uint8).astype(np.float64)
    ug = u.reshape(u.shape[:-1] + (D // group, group))
    return ((ug - z[..., None]) * s[..., None]).reshape(u.shape)


def dequantize_cache_asym(codes, scales, zeros, group, n=None):
    """fp64 ``[B, Hkv, n, D]`` of the first ``n`` cached rows (all rows if None)."""
    if n is None:
        n = codes.shape[2]
    return dequantize_rows_asym(codes[:, :, :n], scales[:, :, :n], zeros[:, :, :n], group)


def attention_asym(q_bits, k_codes, k_scales, k_zeros, v_codes, v_scales, v_zeros, kv_len, softmax_scale, group,
                   causal=False):
    """``attention`` (same definition, fp64) over a cache of asymmetric group-wise rows.

    ``k_codes``/``v_codes`` uint8 ``[B, Hkv, C, D/2]``; scales/zeros ``[B, Hkv, C, D/group]``.
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
            sl = (slice(b, b + 1), slice(g, g + 1))
            kd = dequantize_cache_asym(k_codes[sl], k_scales[sl], k_zeros[sl], group, kv_len)[0, 0]
            vd = dequantize_cache_asym(v_codes[sl], v_scales[sl], v_zeros[sl], group, kv_len)[0, 0]
            for h in range(g * G, (g + 1) * G):
                out[b, h], lse[b, h] = _attend(bf16_bits_to_f64(q_bits[b, h]), kd, vd, scale, causal, kv_len - Sq, 512)
    return out, lse


def cache_order(D: int, tensor: str) -> np.ndarray:
    """Element stored at nibble slot n (slot n = nibble n % 8 of dword n // 8 of a row)."""
    if D not in (64, 128):
        raise ValueError("head dim must be 64 or 128")
    KK = D // 32
    order = np.empty(D, np.int64)
    for w in range(D // 8):
        for i in range(8):
            if tensor == "k":
                j, k = divmod(w, KK)               # dword KK j + k holds chunk 4 k + j
                elem = 8 * (4 * k + j) + i
            elif tensor == "v":
                if D == 128:
                    elem = 16 * i + w              # nibble p = i, lane w
                else:
                    elem = 16 * (i % 4) + w + 8 * (i // 4)
            else:
                raise ValueError("tensor must be 'k' or 'v'")
            order[8 * w + i] = elem
    return order


def _pack_u(u: np.ndarray) -> np.ndarray:
    return (u[..., 0::2] | (u[..., 1::2] << np.uint8(4))).astype(np.uint8)


def to_cache_order(codes: np.ndarray, tensor: str) -> np.ndarray:
    """Packed rows in element order -> the same nibbles in the cache's row order."""
    u = unpack_asym(codes)
    return np.ascontiguousarray(_pack_u(u[..., cache_order(u.shape[-1], tensor)]))


def from_cache_order(codes: np.ndarray, tensor: str) -> np.ndarray:
    """Rows in the cache's order -> packed rows in element order."""
    u = unpack_asym(codes)
    D = u.shape[-1]
    out = np.empty_like(u)
    out[..., cache_order(D, tensor)] = u
    return np.ascontiguousarray(_pack_u(out))

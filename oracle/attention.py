"""fp64 attention oracle over a dequantized int4 KV cache (TEST INFRASTRUCTURE ONLY).

Follows:

* TurboAttention (arXiv 2412.08585) §2.1: attention runs per (batch, head);
  prefill caches K/V, each decode step appends its k/v and its query attends
  the whole updated cache.
* Same paper §2.2 (Equation 2, whose display is lost in the text; its prose
  names the three steps): S = Q K^T, P = softmax(S) row-wise, H = P V.
  FlashAttention (same section, and the FlashAttention entry of the related
  list on the QFlash page) is an exact reformulation of that result, so the
  oracle is the plain, untiled definition.
* "Quantized Cross-Attention ..." §4.1: K/V come from the quantized cache and
  the output is fp32 ``[batch, heads, seq_q, dim]`` (kept here in fp64).

Readings where the pages are silent: query head ``h`` uses KV head
``h // (Hq // Hkv)`` (contiguous GQA groups, as in Llama-3-8B's 8 KV heads);
a causal mask is bottom-right aligned (query row ``i`` of ``Sq`` is token
``kv_len - Sq + i`` and sees keys ``j <= i + kv_len - Sq``); the softmax
scale is the fp32 value the caller passes, widened exactly to fp64.

Everything is fp64 with numpy: dequantize (exact), ``S = Q K^T * scale``
(BLAS matmul), two-pass softmax (row max, exp, row sum, divide), ``O = P V``.
Query rows are processed in chunks only to bound memory.
"""
from __future__ import annotations

import numpy as np

from .quantize import dequantize_cache

__all__ = ["attention", "attention_partial", "lse_merge", "bf16_bits_to_f64"]


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact fp64 value of bfloat16 bit patterns."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _attend(qd, kd, vd, scale, causal, offset, chunk, row_ids=None):
    """Plain attention for one (batch, head): qd [n, D], kd/vd [L, D] fp64.

    ``row_ids`` are the query row indices of the rows of ``qd`` (default
    0..n-1); ``offset`` = kv_len - Sq (bottom-right causal alignment).
    Returns (O [n, D], LSE [n]) with LSE the natural-log log-sum-exp of the
    scaled scores over visible keys.
    """
    Sq = qd.shape[0]
    L = kd.shape[0]
    if row_ids is None:
        row_ids = np.arange(Sq)
    out = np.empty((Sq, qd.shape[1]), dtype=np.float64)
    lse = np.empty(Sq, dtype=np.float64)
    for r0 in range(0, Sq, chunk):
        r1 = min(Sq, r0 + chunk)
        s = (qd[r0:r1] @ kd.T) * scale
        if causal:
            rows = np.asarray(row_ids[r0:r1])[:, None]
            cols = np.arange(L)[None, :]
            s = np.where(cols <= rows + offset, s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        e = np.exp(s - m)
        l = np.sum(e, axis=1, keepdims=True)
        out[r0:r1] = (e / l) @ vd
        lse[r0:r1] = (m + np.log(l))[:, 0]
    return out, lse


def attention(q_bits, k_codes, k_scales, v_codes, v_scales, kv_len, softmax_scale,
              causal=False, heads=None, rows=None, chunk=512):
    """Attention of bf16 queries over the first ``kv_len`` rows of an int4 cache.

    q_bits   uint16 bf16 bits ``[B, Hq, Sq, D]``
    k_codes  uint8 ``[B, Hkv, C, D/2]``, k_scales uint16 fp16 bits ``[B, Hkv, C]``
    v_codes, v_scales: same for V
    heads    optional iterable of (b, h) pairs to compute (others are NaN)
    rows     optional sorted query row indices to compute (others are NaN);
             each row is computed exactly as in the full result

    Returns ``(out, lse)``: fp64 ``[B, Hq, Sq, D]`` and ``[B, Hq, Sq]``.
    """
    B, Hq, Sq, D = q_bits.shape
    Hkv = k_codes.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if causal and Sq > kv_len:
        raise ValueError("causal attention needs Sq <= kv_len")
    scale = float(np.float32(softmax_scale))
    out = np.full((B, Hq, Sq, D), np.nan)
    lse = np.full((B, Hq, Sq), np.nan)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    heads = list(heads)
    cache = {}
    for b, h in heads:
        g = h // G
        if (b, g) not in cache:
            kd = dequantize_cache(k_codes[b:b + 1, g:g + 1], k_scales[b:b + 1, g:g + 1], kv_len)[0, 0]
            vd = dequantize_cache(v_codes[b:b + 1, g:g + 1], v_scales[b:b + 1, g:g + 1], kv_len)[0, 0]
            cache = {(b, g): (kd, vd)}     # keep one KV head resident at a time
        kd, vd = cache[(b, g)]
        if rows is None:
            qd = bf16_bits_to_f64(q_bits[b, h])
            out[b, h], lse[b, h] = _attend(qd, kd, vd, scale, causal, kv_len - Sq, chunk)
        else:
            idx = np.asarray(rows, dtype=np.int64)
            qd = bf16_bits_to_f64(q_bits[b, h, idx])
            out[b, h, idx], lse[b, h, idx] = _attend(qd, kd, vd, scale, causal, kv_len - Sq, chunk,
                                                     row_ids=idx)
    return out, lse


def attention_partial(q_bits, k_codes, k_scales, v_codes, v_scales, key_lo, key_hi, softmax_scale):
    """Non-causal attention restricted to keys ``[key_lo, key_hi)``.

    Returns ``(O_part, lse_part)`` with ``O_part`` normalized over that key
    range alone; the pair is what one split of a split-K decode produces.
    """
    B, Hq, Sq, D = q_bits.shape
    Hkv = k_codes.shape[1]
    G = Hq // Hkv
    scale = float(np.float32(softmax_scale))
    out = np.empty((B, Hq, Sq, D))
    lse = np.empty((B, Hq, Sq))
    kd = dequantize_cache(k_codes[:, :, key_lo:key_hi], k_scales[:, :, key_lo:key_hi])
    vd = dequantize_cache(v_codes[:, :, key_lo:key_hi], v_scales[:, :, key_lo:key_hi])
    for b in range(B):
        for h in range(Hq):
            qd = bf16_bits_to_f64(q_bits[b, h])
            out[b, h], lse[b, h] = _attend(qd, kd[b, h // G], vd[b, h // G], scale, False, 0, 512)
    return out, lse


def lse_merge(parts):
    """Merge partial results over disjoint key ranges into the full result.

    ``parts`` is a sequence of ``(O_s, lse_s)``.  With ``M = max_s lse_s`` and
    ``w_s = exp(lse_s - M)``: ``O = sum_s w_s O_s / sum_s w_s`` and
    ``LSE = M + log(sum_s w_s)`` (the final normalization by the running max
    and sum that FlashAttention performs, TurboAttention §2.2).
    """
    lses = np.stack([p[1] for p in parts])           # [S, ...]
    outs = np.stack([p[0] for p in parts])           # [S, ..., D]
    M = np.max(lses, axis=0)
    w = np.exp(lses - M)
    den = np.sum(w, axis=0)
    out = np.sum(w[..., None] * outs, axis=0) / den[..., None]
    return out, M + np.log(den)

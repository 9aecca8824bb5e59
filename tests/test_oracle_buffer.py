"""Pins of the INT8 decode-buffer oracle against things other than itself.

* hand-derived codes: ties to even, clamping of outliers at +-127, the zero
  scale, and a universal scale computed with exact fractions,
* the flush of rows whose dequantized values are small integers times a power
  of two: their int4 codes and scale are known in closed form,
* attention over int4 rows followed by INT8 rows equals the (separately
  pinned) int4 attention oracle on a cache holding the same values, and a
  pure-Python scalar brute force on a tiny case,
* invariants: |x - dequant(quant(x))| <= s8 / 2 inside the range.
"""
import math
import struct
from fractions import Fraction

import numpy as np

from oracle import (attention, attention_buffered, buffer_scale, dequantize_int8, flush_rows, quantize_int8,
                    quantize_rows)
from qkv_inputs import f32_to_bf16_bits


def _h(x):
    return struct.unpack("<H", struct.pack("<e", x))[0]


def test_int8_codes_by_hand():
    x = np.array([[0.25, 0.75, -0.75, 1.25, 63.6, 100.0, -100.0, 63.25, -63.75, 0.0]], np.float32)
    c = quantize_int8(x, np.array([0.5], np.float32))
    # x / 0.5 = 0.5 (tie -> 0), 1.5 (-> 2), -1.5 (-> -2), 2.5 (-> 2), 127.2 (-> 127), 200 and -200
    # (clamped), 126.5 (tie -> 126), -127.5 (tie -> -128, clamped to -127), 0
    assert c.tolist() == [[0, 2, -2, 2, 127, 127, -127, 126, -127, 0]]
    assert c.dtype == np.int8
    assert quantize_int8(x, np.array([0.0], np.float32)).tolist() == [[0] * 10]


def test_int8_division_is_fp32():
    # 1/3 is not exact: the quotient is the fp32-rounded one, whose rint is 3 here
    x = np.array([[1.0]], np.float32)
    s = np.array([np.float32(1) / np.float32(3)], np.float32)
    assert quantize_int8(x, s).tolist() == [[3]]


def test_buffer_scale_exact_fraction():
    scales = np.array([[_h(0.5), _h(2.0), _h(1.0), _h(99.0)]], np.uint16)   # row 3 lies past L
    s8 = buffer_scale(scales, 3)
    # 7 * 2.0 / 127, rounded once to fp32 (within half an fp32 ulp of the exact fraction)
    assert s8.dtype == np.float32 and s8.shape == (1,)
    assert abs(Fraction(float(s8[0])) - Fraction(14, 127)) <= Fraction(float(np.spacing(s8[0]))) / 2
    assert buffer_scale(scales, 0).tolist() == [0.0]
    assert buffer_scale(np.zeros((2, 5), np.uint16), 5).tolist() == [0.0, 0.0]


def test_int8_roundtrip_error_bound():
    rng = np.random.default_rng(0)
    s8 = np.float32(0.037)
    x = (rng.uniform(-127, 127, size=(50, 64)) * s8).astype(np.float32)
    c = quantize_int8(x, np.full(50, s8, np.float32))
    err = np.abs(dequantize_int8(c, np.full(50, s8, np.float32)) - x.astype(np.float64))
    assert err.max() <= float(s8) / 2 * (1 + 1e-6)
    # outliers sit at the range end
    big = np.full((1, 4), 1e3, np.float32) * np.array([1, -1, 1, -1], np.float32)
    assert dequantize_int8(quantize_int8(big, np.array([s8])), np.array([s8])).tolist() == \
        [[127 * float(s8), -127 * float(s8), 127 * float(s8), -127 * float(s8)]]


def test_flush_closed_form():
    # codes c with max |c| = 7 and s8 = 2^-3: values c / 8 have absmax 7/8, int4 scale 1/8
    # exactly, int4 codes = c (clamp range [-8, 7] not reached)
    c = np.array([[[-7, 7, 3, -2, 0, 1, -1, 5]]], np.int8)          # [1, T=1, D=8]
    kc, ks = flush_rows(c, np.array([0.125], np.float32))
    assert ks.tolist() == [[_h(0.125)]]
    nib = [v & 0xF for v in c[0, 0].tolist()]
    assert kc[0, 0].tolist() == [nib[2 * i] | (nib[2 * i + 1] << 4) for i in range(4)]
    # codes beyond +-7 in INT8 become coarser int4 codes: 127 * s8 is the absmax
    c2 = np.array([[[127, -64, 32, 0]]], np.int8)
    kc2, ks2 = flush_rows(c2, np.array([1.0], np.float32))
    s4 = np.float16(np.float32(127) / np.float32(7))
    assert ks2.tolist() == [[int(np.array(s4).view(np.uint16))]]
    codes = [int(np.clip(np.rint(np.float32(v) / np.float32(s4)), -8, 7)) for v in (127, -64, 32, 0)]
    nib2 = [v & 0xF for v in codes]
    assert kc2[0, 0].tolist() == [nib2[0] | (nib2[1] << 4), nib2[2] | (nib2[3] << 4)]


def _split_case(seed, B, Hq, Hkv, Sq, L, T, D):
    """An int4 cache of L + T rows whose last T rows of each (b, g) share one
    power-of-two scale, so they are also exact INT8 rows (s8 = that scale)."""
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, Sq, D)).astype(np.float32))
    out = []
    tails = []
    for _ in range(2):
        x = rng.standard_normal((B, Hkv, L + T, D)).astype(np.float32)
        codes, scales = quantize_rows(x)
        ints = rng.integers(-7, 8, size=(B, Hkv, T, D))
        ints[..., 0] = 7                                   # absmax 7 -> int4 scale = the unit exactly
        unit = np.float32(2.0) ** rng.integers(-4, 2, size=(B, Hkv)).astype(np.float32)
        tail_vals = (ints * unit[..., None, None]).astype(np.float32)
        tc, ts = quantize_rows(tail_vals)
        codes[:, :, L:], scales[:, :, L:] = tc, ts
        out += [codes, scales]
        tails.append((ints.astype(np.int8), unit.astype(np.float32)))
    return q, out, tails


def test_buffered_attention_equals_int4_attention():
    B, Hq, Hkv, Sq, L, T, D = 2, 4, 2, 3, 37, 9, 16
    q, (kc, ks, vc, vs), ((kt, ksu), (vt, vsu)) = _split_case(5, B, Hq, Hkv, Sq, L, T, D)
    ref_o, ref_l = attention(q, kc, ks, vc, vs, L + T, 0.25)
    # tail buffers hold more rows than are used
    pad = lambda t: np.concatenate([t, np.full(t.shape[:2] + (5, D), 99, np.int8)], axis=2)
    o, l = attention_buffered(q, kc, ks, vc, vs, L, pad(kt), pad(vt), ksu, vsu, T, 0.25)
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, ref_l, rtol=0, atol=1e-12)
    # no int4 rows at all
    o0, _ = attention_buffered(q, kc, ks, vc, vs, 0, kt, vt, ksu, vsu, T, 0.25)
    kc2, ks2 = kc[:, :, L:], ks[:, :, L:]
    vc2, vs2 = vc[:, :, L:], vs[:, :, L:]
    r0, _ = attention(q, kc2, ks2, vc2, vs2, T, 0.25)
    np.testing.assert_allclose(o0, r0, rtol=0, atol=1e-12)


def test_buffered_attention_brute_force():
    # one query row, one head, two int4 rows (scale 0.5) and two INT8 rows (s8 = 0.25)
    q = f32_to_bf16_bits(np.array([[[[1.0, -2.0]]]], np.float32))
    nib = lambda a, b: (a & 0xF) | ((b & 0xF) << 4)
    kc = np.array([[[[nib(1, 2)], [nib(-3, 0)]]]], np.uint8)
    vc = np.array([[[[nib(2, -1)], [nib(0, 4)]]]], np.uint8)
    s = np.array([[[_h(0.5), _h(0.5)]]], np.uint16)
    kt = np.array([[[[10, -4], [0, 8]]]], np.int8)
    vt = np.array([[[[-6, 2], [12, 1]]]], np.int8)
    s8 = np.array([[0.25]], np.float32)
    o, l = attention_buffered(q, kc, s, vc, s, 2, kt, vt, s8, s8, 2, 0.5)
    keys = [(0.5, 1.0), (-1.5, 0.0), (2.5, -1.0), (0.0, 2.0)]
    vals = [(1.0, -0.5), (0.0, 2.0), (-1.5, 0.5), (3.0, 0.25)]
    sc = [0.5 * (1.0 * k0 - 2.0 * k1) for k0, k1 in keys]
    m = max(sc)
    e = [math.exp(x - m) for x in sc]
    den = math.fsum(e)
    want = [math.fsum(ei * v[d] for ei, v in zip(e, vals)) / den for d in range(2)]
    assert np.allclose(o[0, 0, 0], want, rtol=0, atol=1e-14)
    assert abs(l[0, 0, 0] - (m + math.log(den))) < 1e-14

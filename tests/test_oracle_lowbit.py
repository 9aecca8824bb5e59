"""Pins of the 2- and 3-bit row quantizer oracle against things other than itself.

* hand-derived rows (ties to even, two's complement fields, the 3-bit planes),
* an exact-rational re-derivation of every rounding step on random rows with
  the bit layout written out independently (struct-free shifts on Python ints),
* the 4-bit case equals the pinned int4 quantizer; attention over 2/3-bit
  rows equals the pinned int4 attention oracle on a cache holding the same
  values (a 2- or 3-bit code is a valid int4 code under the same scale),
* invariants: the row maximum maps to +-qmax and |x - s c| <= s/2.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import attention, attention_bits, quantize_rows, quantize_rows_bits, row_bytes, unpack_bits
from qkv_inputs import f32_to_bf16_bits
from test_oracle_quantize import _random_rows, _rn16, _rn32


def _h(x):
    return struct.unpack("<H", struct.pack("<e", x))[0]


def test_row_bytes():
    assert [row_bytes(128, b) for b in (2, 3, 4)] == [32, 48, 64]
    assert [row_bytes(64, b) for b in (2, 3, 4)] == [16, 24, 32]


def test_two_bit_row_by_hand():
    x = np.array([[1.0, -1.0, 0.4, -0.6, 0.5, -0.5, 0.0, 0.2]], np.float32)
    codes, scales = quantize_rows_bits(x, 2)
    # absmax 1, qmax 1: scale 1; codes 1, -1, 0, -1, 0 (tie), 0 (tie), 0, 0
    # two-bit fields 01 11 00 11 | 00 00 00 00 -> 0b11_00_11_01, 0
    assert scales.tolist() == [_h(1.0)]
    assert codes.tolist() == [[0b11001101, 0]]
    assert unpack_bits(codes, 8, 2).tolist() == [[1, -1, 0, -1, 0, 0, 0, 0]]


def test_three_bit_row_by_hand():
    x = np.array([[3.0, -3.0, 1.5, -1.5, 2.5, -0.5, 1.0, -2.0]], np.float32)
    codes, scales = quantize_rows_bits(x, 3)
    # absmax 3, qmax 3: scale 1; codes 3, -3, 2 (tie), -2 (tie), 2 (tie), 0 (tie), 1, -2
    # low two bits 11 01 10 10 | 10 00 01 10; top bits 0 1 0 1 0 0 0 1
    assert scales.tolist() == [_h(1.0)]
    assert codes.tolist() == [[0b10_10_01_11, 0b10_01_00_10, 0b1000_1010]]
    assert unpack_bits(codes, 8, 3).tolist() == [[3, -3, 2, -2, 2, 0, 1, -2]]


def _brute_row(row, bits):
    qmax = 2 ** (bits - 1) - 1
    xs = [Fraction(float(v)) for v in row]
    amax = max(abs(v) for v in xs)
    s16 = _rn16(_rn32(amax / qmax))
    codes = [0] * len(xs)
    if s16 != 0:
        codes = [min(qmax, max(-qmax - 1, round(_rn32(v / s16)))) for v in xs]
    D = len(xs)
    lo = [(c & 3) for c in codes]
    out = bytearray()
    for i in range(D // 4):
        out.append(lo[4 * i] | lo[4 * i + 1] << 2 | lo[4 * i + 2] << 4 | lo[4 * i + 3] << 6)
    if bits == 3:
        for i in range(D // 8):
            out.append(sum(((codes[8 * i + k] >> 2) & 1) << k for k in range(8)))
    return struct.unpack("<H", struct.pack("<e", float(s16)))[0], bytes(out), codes


@pytest.mark.parametrize("bits", [2, 3])
def test_exact_rational_brute_force(bits):
    rng = np.random.default_rng(77 + bits)
    rows = _random_rows(rng, 300, 16)
    codes, scales = quantize_rows_bits(rows, bits)
    for i in range(rows.shape[0]):
        sb, pb, cl = _brute_row(rows[i], bits)
        assert int(scales[i]) == sb, (i, rows[i])
        assert codes[i].tobytes() == pb, (i, rows[i])
        assert unpack_bits(codes[i], 16, bits).tolist() == cl


def test_four_bits_is_the_int4_quantizer():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((50, 64)).astype(np.float32)
    c4, s4 = quantize_rows_bits(x, 4)
    c, s = quantize_rows(x)
    assert np.array_equal(c4, c) and np.array_equal(s4, s)


@pytest.mark.parametrize("bits", [2, 3])
def test_range_and_error_bound(bits):
    rng = np.random.default_rng(bits)
    x = (rng.standard_normal((2000, 64)) * 3.0).astype(np.float32)
    c, s = quantize_rows_bits(x, bits)
    codes = unpack_bits(c, 64, bits).astype(np.int64)
    qmax = 2 ** (bits - 1) - 1
    top = codes[np.arange(x.shape[0]), np.argmax(np.abs(x), axis=1)]
    assert np.all(np.abs(top) == qmax)
    assert codes.min() >= -qmax - 1 and codes.max() <= qmax
    sv = s.view(np.float16).astype(np.float64)[:, None]
    err = np.abs(x.astype(np.float64) - sv * codes)
    assert np.all(err <= sv / 2 * (1 + 2.0 ** -10))


def _as_int4(codes, D, bits):
    """Re-pack b-bit codes as int4 nibbles (independent of the oracle's packer)."""
    c = unpack_bits(codes, D, bits).astype(np.int64) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_attention_equals_int4_attention_on_same_values(bits, causal):
    rng = np.random.default_rng(bits * 10 + causal)
    B, Hq, Hkv, Sq, L, D = 2, 4, 2, 3, 21, 16
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, Sq, D)).astype(np.float32))
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    kc, ks = quantize_rows_bits(k, bits)
    vc, vs = quantize_rows_bits(v, bits)
    o, l = attention_bits(q, kc, ks, vc, vs, L, 0.3, bits, causal=causal)
    ro, rl = attention(q, _as_int4(kc, D, bits), ks, _as_int4(vc, D, bits), vs, L, 0.3, causal=causal)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, rl, rtol=0, atol=1e-12)

"""Pins of the quantizer oracle against things other than itself.

* hand-derived worked examples (tests/golden/quantizer_rows.txt),
* an exact-rational re-derivation of every rounding step (brute force with
  ``fractions.Fraction``, no numpy floating point), on random rows that
  include exact ties and subnormal scales,
* invariants: idempotence on dequantized rows, the absmax element maps to +-7,
  the rounding-error bound, untouched rows outside the append range.
"""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import quantize_rows, dequantize_rows, quantize_append

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantizer_rows.txt")


def _load_golden():
    cases, cur = [], {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            if key == "row":
                cur = {"row": np.array([float(t) for t in val.split()], dtype=np.float32)}
            elif key == "scale":
                cur["scale"] = int(val, 16)
            elif key == "bytes":
                cur["bytes"] = bytes(int(t, 16) for t in val.split())
                cases.append(cur)
    return cases


GOLDEN_CASES = _load_golden()


def test_golden_file_has_cases():
    assert len(GOLDEN_CASES) == 8


@pytest.mark.parametrize("case", GOLDEN_CASES, ids=[str(i) for i in range(len(GOLDEN_CASES))])
def test_golden_rows(case):
    codes, scale = quantize_rows(case["row"][None, :])
    assert int(scale[0]) == case["scale"]
    assert codes[0].tobytes() == case["bytes"]


# ---------------------------------------------------------------- exact brute force

def _exact(x32: np.float32) -> Fraction:
    return Fraction(float(x32))


def _round_binary(x: Fraction, p: int, emin: int) -> Fraction:
    """Round to nearest, ties to even, into a binary format with a p-bit
    significand and minimum normal exponent emin (gradual underflow)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (p - 1))
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def _rn32(x):
    return _round_binary(x, 24, -126)


def _rn16(x):
    return _round_binary(x, 11, -14)


def _fp16_bits(v: Fraction) -> int:
    return struct.unpack("<H", struct.pack("<e", float(v)))[0]


def _brute_row(row):
    xs = [_exact(v) for v in row]
    amax = max(abs(v) for v in xs)
    s16 = _rn16(_rn32(amax / 7))
    if s16 == 0:
        codes = [0] * len(xs)
    else:
        codes = []
        for v in xs:
            r = _rn32(v / s16)
            c = round(r)                     # Fraction.__round__: half to even
            codes.append(min(7, max(-8, c)))
    packed = bytes(((codes[2 * i] & 0xF) | ((codes[2 * i + 1] & 0xF) << 4)) for i in range(len(codes) // 2))
    return _fp16_bits(s16), packed


def _random_rows(rng, n, D):
    rows = []
    for _ in range(n):
        kind = rng.integers(0, 4)
        if kind == 0:      # generic magnitudes over a wide exponent range
            r = rng.standard_normal(D) * 2.0 ** rng.integers(-30, 12)
        elif kind == 1:    # exact ties: amax = 7 s for an fp16 s, values (k + 1/2) s
            s = np.float16(abs(rng.standard_normal()) * 2.0 ** rng.integers(-12, 8))
            if s == 0:
                s = np.float16(1.0)
            ks = rng.integers(-7, 7, size=D).astype(np.float64) + 0.5
            ks[0] = 7.0
            r = ks * float(s)
        elif kind == 2:    # subnormal-scale rows (clamp can bind)
            r = rng.standard_normal(D) * 2.0 ** rng.integers(-27, -20)
        else:              # near-zero and zero elements mixed in
            r = rng.standard_normal(D) * (rng.random(D) < 0.5)
        rows.append(np.asarray(r, dtype=np.float32))
    return np.stack(rows)


def test_exact_rational_brute_force():
    rng = np.random.default_rng(1234)
    rows = _random_rows(rng, 300, 8)
    codes, scales = quantize_rows(rows)
    for i in range(rows.shape[0]):
        sb, pb = _brute_row(rows[i])
        assert int(scales[i]) == sb, (i, rows[i])
        assert codes[i].tobytes() == pb, (i, rows[i])


# ---------------------------------------------------------------- invariants

def test_idempotent_on_dequantized_rows():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4000, 64)).astype(np.float32)
    c, s = quantize_rows(x)
    sv = s.view(np.float16)
    assert np.all(np.abs(sv.astype(np.float32)) >= np.float32(2.0 ** -14))   # normal scales
    deq = dequantize_rows(c, s)
    assert np.all(deq.astype(np.float32).astype(np.float64) == deq)          # exact in fp32
    c2, s2 = quantize_rows(deq.astype(np.float32))
    assert np.array_equal(c, c2) and np.array_equal(s, s2)


def _codes(c):
    lo = (c & 0xF).astype(np.int16)
    hi = (c >> 4).astype(np.int16)
    out = np.empty(c.shape[:-1] + (2 * c.shape[-1],), np.int16)
    out[..., 0::2], out[..., 1::2] = lo, hi
    return np.where(out >= 8, out - 16, out)


def test_absmax_maps_to_seven_and_error_bound():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((3000, 128)) * 3.0).astype(np.float32)
    c, s = quantize_rows(x)
    codes = _codes(c)
    idx = np.argmax(np.abs(x), axis=1)
    top = codes[np.arange(x.shape[0]), idx]
    assert np.all(np.abs(top) == 7)
    assert np.all(np.sign(top) == np.sign(x[np.arange(x.shape[0]), idx]))
    assert codes.min() >= -7 and codes.max() <= 7          # normal scales never reach -8
    sv = s.view(np.float16).astype(np.float64)[:, None]
    err = np.abs(x.astype(np.float64) - sv * codes)
    assert np.all(err <= sv / 2 * (1 + 2.0 ** -10))


def test_append_touches_only_its_rows():
    rng = np.random.default_rng(9)
    B, H, C, D, T, pos = 2, 3, 20, 16, 5, 7
    codes = np.full((B, H, C, D // 2), 0xA5, np.uint8)
    scales = np.full((B, H, C), 0xA5A5, np.uint16)
    src = rng.standard_normal((B, H, T, D)).astype(np.float32)
    quantize_append(src, codes, scales, pos)
    qc, qs = quantize_rows(src)
    assert np.array_equal(codes[:, :, pos:pos + T], qc)
    assert np.array_equal(scales[:, :, pos:pos + T], qs)
    assert np.all(codes[:, :, :pos] == 0xA5) and np.all(codes[:, :, pos + T:] == 0xA5)
    assert np.all(scales[:, :, :pos] == 0xA5A5) and np.all(scales[:, :, pos + T:] == 0xA5A5)
    with pytest.raises(ValueError):
        quantize_append(src, codes, scales, C - T + 1)


def test_dequantize_exact_values():
    # nibble -> value table written out: two's complement, low nibble first
    c = np.array([[0x10, 0x98, 0xF7, 0x8E]], np.uint8)
    s = np.array([0x4000], np.uint16)           # 2.0
    v = dequantize_rows(c, s)[0]
    assert list(v) == [0.0, 2.0, -16.0, -14.0, 14.0, -2.0, -4.0, -16.0]
    assert math.isclose(float(np.float16(0.5)), 0.5)

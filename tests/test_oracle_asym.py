"""Pins of the asymmetric group-wise int4 oracle against things other than itself.

* a hand-derived row (two groups: one straddling zero, one all positive),
* an exact-rational re-derivation of every rounding step on random rows
  (exact ties, all-positive and all-negative groups, zero groups, subnormal
  scales), with the packing written out independently,
* invariants: codes and zero points in [0, 15], zero maps to zero exactly,
  the rounding-error bound,
* symmetric int4 rows embedded as asymmetric rows (zero point 8, codes + 8,
  one group per row): the same values, and attention equal to the pinned
  int4 attention oracle,
* the cache's row orders: hand-checked slots, a permutation, a round trip.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import (attention, attention_asym, dequantize_rows, dequantize_rows_asym, quantize_rows,
                    quantize_rows_asym, unpack_asym)
from qkv_inputs import f32_to_bf16_bits
from test_oracle_quantize import _exact, _round_binary


def _rn32(x):
    return _round_binary(x, 24, -126)


def _rn16(x):
    return _round_binary(x, 11, -14)


def _h(v):
    return struct.unpack("<H", struct.pack("<e", float(v)))[0]


def test_row_by_hand():
    x = np.array([[-1.5, 0.0, 3.0, 1.0, 0.25, 0.5, 1.0, 0.75]], np.float32)
    codes, scales, zeros = quantize_rows_asym(x, 4)
    # group 0: lo -1.5, hi 3.0, s = fp16(4.5/15) = 0.30004883 (0x34CD);
    #          z = rint(1.5 / s) = rint(4.9992) = 5; u = rint(x/s) + 5 = 0, 5, 15 (10 + 5), 8 (3 + 5)
    # group 1: all positive, lo = 0, hi 1.0, s = fp16(1/15) = 0.066650 (0x2C44); z = 0;
    #          u = rint(3.751) = 4, rint(7.502) = 8, rint(15.004) = 15, rint(11.253) = 11
    assert scales.tolist() == [[0x34CD, 0x2C44]]
    assert zeros.tolist() == [[5, 0]]
    assert unpack_asym(codes).tolist() == [[0, 5, 15, 8, 4, 8, 15, 11]]
    assert codes.tolist() == [[0x50, 0x8F, 0x84, 0xBF]]
    s0 = float(np.float16(0.3))
    want = [s0 * (u - 5) for u in (0, 5, 15, 8)] + [float(np.float16(1 / 15)) * u for u in (4, 8, 15, 11)]
    assert dequantize_rows_asym(codes, scales, zeros, 4).tolist() == [want]


def test_zero_groups():
    x = np.zeros((2, 8), np.float32)
    x[1, 4:] = [1e-3, -2e-3, 0.0, 5e-4]
    codes, scales, zeros = quantize_rows_asym(x, 4)
    assert scales[0].tolist() == [0, 0] and zeros[0].tolist() == [0, 0] and codes[0].tolist() == [0, 0, 0, 0]
    assert scales[1, 0] == 0 and zeros[1, 0] == 0 and unpack_asym(codes)[1, :4].tolist() == [0, 0, 0, 0]
    assert scales[1, 1] != 0


def _brute_group(xs):
    """Scale bits, zero point and codes of one group, every step in exact rationals."""
    lo = min([Fraction(0)] + xs)
    hi = max([Fraction(0)] + xs)
    s = _rn16(_rn32(_rn32(hi - lo) / 15))
    if s == 0:
        return _h(0.0), 0, [0] * len(xs)
    z = min(15, max(0, round(_rn32(-lo / s))))            # round(): half to even
    us = [min(15, max(0, round(_rn32(v / s)) + z)) for v in xs]
    return _h(s), z, us


def _asym_rows(rng, n, D):
    rows = []
    for _ in range(n):
        kind = rng.integers(0, 6)
        if kind == 0:      # generic magnitudes over a wide exponent range
            r = rng.standard_normal(D) * 2.0 ** rng.integers(-30, 12)
        elif kind == 1:    # exact ties: range 15 s for an fp16 s, values (k + 1/2) s
            s = float(np.float16(abs(rng.standard_normal()) * 2.0 ** rng.integers(-10, 6)) or 1.0)
            a = int(rng.integers(1, 14))
            k = rng.integers(-a, 15 - a, size=D).astype(np.float64) + 0.5
            k[0], k[1] = -a, 15 - a
            r = k * s
        elif kind == 2:    # all positive
            r = np.abs(rng.standard_normal(D)) + 0.5
        elif kind == 3:    # all negative
            r = -np.abs(rng.standard_normal(D)) * 3.0 - 0.1
        elif kind == 4:    # subnormal scales
            r = rng.standard_normal(D) * 2.0 ** rng.integers(-27, -20)
        else:              # zeros mixed in, some groups all zero
            r = rng.standard_normal(D) * (rng.random(D) < 0.5)
            r[: D // 2] = 0.0
        rows.append(np.asarray(r, dtype=np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("group", [4, 8, 16])
def test_exact_rational_brute_force(group):
    rng = np.random.default_rng(300 + group)
    D = 16
    rows = _asym_rows(rng, 300, D)
    codes, scales, zeros = quantize_rows_asym(rows, group)
    for i in range(rows.shape[0]):
        us_all = []
        for g0 in range(0, D, group):
            sb, z, us = _brute_group([_exact(v) for v in rows[i, g0:g0 + group]])
            assert int(scales[i, g0 // group]) == sb, (i, g0, rows[i])
            assert int(zeros[i, g0 // group]) == z, (i, g0, rows[i])
            us_all += us
        packed = bytes(us_all[2 * k] | (us_all[2 * k + 1] << 4) for k in range(D // 2))
        assert codes[i].tobytes() == packed, (i, rows[i])


@pytest.mark.parametrize("group", [32, 64, 128])
def test_invariants(group):
    rng = np.random.default_rng(group)
    x = (rng.standard_normal((500, 128)) * 2.0).astype(np.float32)
    x[::7] += 3.0                      # rows whose groups sit off zero
    x[3, :group] = 0.0
    codes, scales, zeros = quantize_rows_asym(x, group)
    u = unpack_asym(codes)
    assert u.max() <= 15 and zeros.max() <= 15
    xq = dequantize_rows_asym(codes, scales, zeros, group)
    # zero is exactly representable: x = 0 dequantizes to 0
    xz = x.copy()
    xz[:, ::5] = 0.0
    cz, sz, zz = quantize_rows_asym(xz, group)
    assert np.all(dequantize_rows_asym(cz, sz, zz, group)[:, ::5] == 0.0)
    # error bound: half a step, plus the end-of-range clamp a rounded-down scale can cause
    s = np.repeat(scales.view(np.float16).astype(np.float64), group, axis=-1)
    assert np.all(np.abs(xq - x.astype(np.float64)) <= s * (0.5 + 16 * 2.0 ** -11))


def _embed(codes4):
    """Symmetric int4 nibbles c -> unsigned asymmetric codes c + 8 (zero point 8)."""
    c = codes4.astype(np.int64)
    lo = ((c & 15) ^ 8) & 15
    hi = (((c >> 4) & 15) ^ 8) & 15
    return (lo | (hi << 4)).astype(np.uint8)


def test_symmetric_rows_embed():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((40, 64)).astype(np.float32)
    c, s = quantize_rows(x)
    z = np.full((40, 1), 8, np.uint8)
    np.testing.assert_array_equal(dequantize_rows_asym(_embed(c), s[:, None], z, 64), dequantize_rows(c, s))


@pytest.mark.parametrize("causal", [False, True])
def test_attention_equals_int4_attention_on_embedded_rows(causal):
    rng = np.random.default_rng(11 + causal)
    B, Hq, Hkv, Sq, L, D = 2, 4, 2, 3, 19, 16
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, Sq, D)).astype(np.float32))
    kc, ks = quantize_rows(rng.standard_normal((B, Hkv, L, D)).astype(np.float32))
    vc, vs = quantize_rows(rng.standard_normal((B, Hkv, L, D)).astype(np.float32))
    z = np.full((B, Hkv, L, 1), 8, np.uint8)
    o, l = attention_asym(q, _embed(kc), ks[..., None], z, _embed(vc), vs[..., None], z, L, 0.3, D, causal=causal)
    ro, rl = attention(q, kc, ks, vc, vs, L, 0.3, causal=causal)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, rl, rtol=0, atol=1e-12)


def test_cache_order_by_hand():
    from oracle import cache_order
    k128 = cache_order(128, "k").reshape(16, 8)
    assert k128[1].tolist() == list(range(32, 40))      # dword 1 = chunk 4 (k = 1, j = 0)
    assert k128[4].tolist() == list(range(8, 16))       # dword 4 = chunk 1 (k = 0, j = 1)
    assert k128[15].tolist() == list(range(120, 128))
    k64 = cache_order(64, "k").reshape(8, 8)
    assert k64[1].tolist() == list(range(32, 40)) and k64[2].tolist() == list(range(8, 16))
    v128 = cache_order(128, "v").reshape(16, 8)
    assert v128[0].tolist() == [0, 16, 32, 48, 64, 80, 96, 112]
    assert v128[5].tolist() == [5, 21, 37, 53, 69, 85, 101, 117]
    v64 = cache_order(64, "v").reshape(8, 8)
    assert v64[0].tolist() == [0, 16, 32, 48, 8, 24, 40, 56]
    assert v64[7].tolist() == [7, 23, 39, 55, 15, 31, 47, 63]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("tensor", ["k", "v"])
def test_cache_order_round_trip(D, tensor):
    from oracle import cache_order, from_cache_order, to_cache_order
    assert sorted(cache_order(D, tensor).tolist()) == list(range(D))
    rng = np.random.default_rng(D)
    c = rng.integers(0, 256, size=(5, 3, D // 2), dtype=np.uint8)
    t = to_cache_order(c, tensor)
    assert np.array_equal(from_cache_order(t, tensor), c)
    # slot n of the stored row holds element cache_order[n]
    assert np.array_equal(unpack_asym(t), unpack_asym(c)[..., cache_order(D, tensor)])


def _py_asym_row(codes_row, scale_bits, zeros, group):
    """One packed row in element order -> its values, scalar Python (s (u - z) per group)."""
    from test_oracle_attention import _py_f16
    us = []
    for byte in codes_row:
        us += [int(byte) & 0xF, int(byte) >> 4]
    return [_py_f16(scale_bits[e // group]) * (u - int(zeros[e // group])) for e, u in enumerate(us)]


@pytest.mark.parametrize("group", [4, 8])
@pytest.mark.parametrize("Hq,Hkv,Sq,L,causal", [(4, 2, 3, 12, False), (4, 2, 5, 12, True), (6, 3, 2, 9, True)])
def test_attention_asym_brute_force(group, Hq, Hkv, Sq, L, causal):
    """Several groups per row (D = 16): pure-Python scalar loops (math.exp,
    math.fsum, struct-decoded fp16 scales and bf16 queries) against the oracle."""
    import math
    from test_oracle_attention import _py_bf16
    rng = np.random.default_rng(group * 100 + Hq + Sq + L + causal)
    B, D = 2, 16
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, Sq, D)).astype(np.float32))
    k = (rng.standard_normal((B, Hkv, L + 2, D)) * rng.uniform(0.2, 3.0, size=(1, 1, 1, D)) + 0.5).astype(np.float32)
    v = (rng.standard_normal((B, Hkv, L + 2, D)) - 0.3).astype(np.float32)
    kc, ks, kz = quantize_rows_asym(k, group)
    vc, vs, vz = quantize_rows_asym(v, group)
    assert len(set(kz.ravel().tolist())) > 1 and len(set(ks[0, 0, 0].tolist())) > 1   # zero points and scales vary
    scale = float(np.float32(0.41))
    o, l = attention_asym(q, kc, ks, kz, vc, vs, vz, L, scale, group, causal=causal)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            g = h // G
            K = [_py_asym_row(kc[b, g, j], ks[b, g, j], kz[b, g, j], group) for j in range(L)]
            V = [_py_asym_row(vc[b, g, j], vs[b, g, j], vz[b, g, j], group) for j in range(L)]
            for i in range(Sq):
                qi = [_py_bf16(q[b, h, i, d]) for d in range(D)]
                vis = [j for j in range(L) if (not causal) or j <= i + L - Sq]
                sc = [math.fsum(qi[d] * K[j][d] for d in range(D)) * scale for j in vis]
                m = max(sc)
                e = [math.exp(x - m) for x in sc]
                den = math.fsum(e)
                for d in range(D):
                    want = math.fsum(e[t] * V[j][d] for t, j in enumerate(vis)) / den
                    assert abs(o[b, h, i, d] - want) < 1e-12
                assert abs(l[b, h, i] - (m + math.log(den))) < 1e-12

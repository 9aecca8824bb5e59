"""Pins of the fp64 attention oracle against things other than itself.

* brute force: pure-Python scalar loops (math.exp / math.fsum, dequantization
  re-done from the nibble bits with struct) on tiny inputs, GQA and causal,
* closed forms: zero query or identical keys give the mean of the visible V
  rows (pins bottom-right causal alignment), a single key gives that row,
  a dominant key gives its row, per-group constant V pins the GQA head map,
  two keys with a known score gap give known weights (pins the scale and the
  natural-base exponential), LSE of equal scores is s + ln(n),
* invariants: KV-permutation invariance, split-merge invariance, GQA equals
  MHA with repeated KV heads, softmax rows sum to one.
"""
import math
import struct

import numpy as np
import pytest

from oracle import attention, attention_partial, lse_merge, quantize_rows
from qkv_inputs import f32_to_bf16_bits


def _cache(k, v):
    kc, ks = quantize_rows(k)
    vc, vs = quantize_rows(v)
    return kc, ks, vc, vs


def _rand_case(seed, B, Hq, Hkv, Sq, L, D, C=None):
    rng = np.random.default_rng(seed)
    C = C or L
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, Sq, D)).astype(np.float32))
    k = rng.standard_normal((B, Hkv, C, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, C, D)).astype(np.float32)
    return (q,) + _cache(k, v)


def _pack_codes(ints):
    """int array [..., D] of values in [-8, 7] -> packed bytes (independent of the oracle)."""
    ints = np.asarray(ints, dtype=np.int64)
    n = ints & 0xF
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def _h(x):
    return struct.unpack("<H", struct.pack("<e", x))[0]


# ------------------------------------------------------------------ brute force

def _py_bf16(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _py_f16(bits):
    return struct.unpack("<e", struct.pack("<H", int(bits)))[0]


def _py_row(codes_row, scale_bits):
    s = _py_f16(scale_bits)
    out = []
    for byte in codes_row:
        for nib in (int(byte) & 0xF, int(byte) >> 4):
            out.append(s * (nib - 16 if nib >= 8 else nib))
    return out


def _brute(q, kc, ks, vc, vs, L, scale, causal):
    B, Hq, Sq, D = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Sq, D))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            K = [_py_row(kc[b, g, j], ks[b, g, j]) for j in range(L)]
            V = [_py_row(vc[b, g, j], vs[b, g, j]) for j in range(L)]
            for i in range(Sq):
                qi = [_py_bf16(q[b, h, i, d]) for d in range(D)]
                vis = [j for j in range(L) if (not causal) or j <= i + L - Sq]
                sc = [math.fsum(qi[d] * K[j][d] for d in range(D)) * scale for j in vis]
                m = max(sc)
                e = [math.exp(x - m) for x in sc]
                den = math.fsum(e)
                for d in range(D):
                    out[b, h, i, d] = math.fsum(e[t] * V[j][d] for t, j in enumerate(vis)) / den
                lse[b, h, i] = m + math.log(den)
    return out, lse


@pytest.mark.parametrize("Hq,Hkv,Sq,L,causal", [
    (4, 2, 1, 1, False), (4, 2, 3, 16, False), (4, 2, 5, 16, True), (2, 2, 4, 4, True),
    (6, 3, 2, 9, False), (4, 1, 7, 11, True),
])
def test_brute_force(Hq, Hkv, Sq, L, causal):
    q, kc, ks, vc, vs = _rand_case(11 + Hq + Sq + L, 2, Hq, Hkv, Sq, L, 8, C=L + 3)
    scale = float(np.float32(0.37))
    o, l = attention(q, kc, ks, vc, vs, L, scale, causal)
    ob, lb = _brute(q, kc, ks, vc, vs, L, scale, causal)
    assert np.max(np.abs(o - ob)) < 1e-12
    assert np.max(np.abs(l - lb)) < 1e-12


# ------------------------------------------------------------------ closed forms

def _int_cache(kints, vints, kscale=1.0, vscale=1.0):
    kc = _pack_codes(kints)
    vc = _pack_codes(vints)
    ks = np.full(kc.shape[:-1], _h(kscale), np.uint16)
    vs = np.full(vc.shape[:-1], _h(vscale), np.uint16)
    return kc, ks, vc, vs


def test_zero_query_gives_mean_of_visible_values_bottom_right():
    rng = np.random.default_rng(3)
    B, H, L, D, Sq = 1, 1, 12, 4, 5
    kints = rng.integers(-8, 8, size=(B, H, L, D))
    vints = rng.integers(-8, 8, size=(B, H, L, D))
    kc, ks, vc, vs = _int_cache(kints, vints)
    q = np.zeros((B, H, Sq, D), np.uint16)          # bf16 +0.0
    o, lse = attention(q, kc, ks, vc, vs, L, 1.0, causal=True)
    for i in range(Sq):
        n = L - Sq + i + 1                          # row i is token L-Sq+i
        assert np.allclose(o[0, 0, i], vints[0, 0, :n].mean(axis=0), atol=1e-14, rtol=0)
        assert abs(lse[0, 0, i] - math.log(n)) < 1e-14
    o2, _ = attention(q, kc, ks, vc, vs, L, 1.0, causal=False)
    assert np.allclose(o2[0, 0], vints[0, 0].mean(axis=0), atol=1e-14, rtol=0)


def test_identical_keys_give_prefix_means_and_lse():
    rng = np.random.default_rng(4)
    B, H, L, D, Sq = 1, 2, 9, 8, 9
    krow = rng.integers(-8, 8, size=D)
    kints = np.broadcast_to(krow, (B, H, L, D))
    vints = rng.integers(-8, 8, size=(B, H, L, D))
    kc, ks, vc, vs = _int_cache(kints, vints, kscale=0.5)
    qf = rng.standard_normal((B, H, Sq, D)).astype(np.float32)
    q = f32_to_bf16_bits(qf)
    o, lse = attention(q, kc, ks, vc, vs, L, 0.25, causal=True)
    for h in range(H):
        for i in range(Sq):
            assert np.allclose(o[0, h, i], vints[0, h, :i + 1].mean(axis=0), atol=1e-13, rtol=0)
            qv = (q[0, h, i].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            s0 = float(np.dot(qv, 0.5 * krow)) * 0.25
            assert abs(lse[0, h, i] - (s0 + math.log(i + 1))) < 1e-12


def test_single_key_and_causal_row0():
    q, kc, ks, vc, vs = _rand_case(5, 1, 2, 2, 1, 1, 16)
    o, _ = attention(q, kc, ks, vc, vs, 1, 0.125)
    assert np.array_equal(o[0, 0, 0], np.array(_py_row(vc[0, 0, 0], vs[0, 0, 0])))
    q, kc, ks, vc, vs = _rand_case(6, 1, 1, 1, 6, 6, 8)
    o, _ = attention(q, kc, ks, vc, vs, 6, 0.3, causal=True)
    assert np.array_equal(o[0, 0, 0], np.array(_py_row(vc[0, 0, 0], vs[0, 0, 0])))


def test_dominant_key():
    B, H, L, D = 1, 1, 7, 8
    kints = np.zeros((B, H, L, D), int)
    kints[0, 0, 4, :] = 7                     # key 4 aligned with q
    vints = np.arange(L * D).reshape(B, H, L, D) % 15 - 7
    kc, ks, vc, vs = _int_cache(kints, vints, kscale=4.0)
    q = f32_to_bf16_bits(np.ones((B, H, 1, D), np.float32))
    # score gap = 8 * 7 * 4 * scale = 224 * 0.25 = 56 (>= 50)
    o, _ = attention(q, kc, ks, vc, vs, L, 0.25)
    assert np.allclose(o[0, 0, 0], vints[0, 0, 4], rtol=0, atol=1e-15 * 8)


def test_two_keys_known_weights():
    # q = e0, k0 = 0, k1 = 3 * 0.5 * e0 -> raw score gap 1.5; scale x gives gap 1.5 x
    D = 8
    kints = np.zeros((1, 1, 2, D), int)
    kints[0, 0, 1, 0] = 3
    vints = np.zeros((1, 1, 2, D), int)
    vints[0, 0, 0, :] = 2
    vints[0, 0, 1, :] = -4
    kc, ks, vc, vs = _int_cache(kints, vints, kscale=0.5)
    qf = np.zeros((1, 1, 1, D), np.float32)
    qf[..., 0] = 1.0
    q = f32_to_bf16_bits(qf)
    x = float(np.float32(math.log(3.0) / 1.5))
    o, lse = attention(q, kc, ks, vc, vs, 2, x)
    gap = 1.5 * x
    w1 = math.exp(gap) / (1 + math.exp(gap))            # ~ 3/4
    assert abs(w1 - 0.75) < 1e-7
    assert np.allclose(o[0, 0, 0], (1 - w1) * 2 + w1 * -4, atol=1e-14, rtol=0)
    assert abs(lse[0, 0, 0] - math.log(1 + math.exp(gap))) < 1e-14


def test_gqa_head_map_is_contiguous_groups():
    rng = np.random.default_rng(6)
    B, Hq, Hkv, L, D = 2, 6, 3, 5, 8
    kints = rng.integers(-8, 8, size=(B, Hkv, L, D))
    vints = np.ones((B, Hkv, L, D), int)
    kc = _pack_codes(kints)
    vc = _pack_codes(vints)
    ks = np.full((B, Hkv, L), _h(1.0), np.uint16)
    vs = np.empty((B, Hkv, L), np.uint16)
    for g in range(Hkv):
        vs[:, g, :] = _h(float(g + 1))            # V of KV head g is the constant g+1
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, 3, D)).astype(np.float32))
    o, _ = attention(q, kc, ks, vc, vs, L, 0.2)
    G = Hq // Hkv
    for h in range(Hq):
        assert np.allclose(o[:, h], h // G + 1, atol=1e-14, rtol=0)


# ------------------------------------------------------------------ invariants

def test_rows_sum_to_one():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, Sq, L, D = 1, 4, 2, 6, 30, 16
    kc, ks, _, _ = _rand_case(12, B, Hq, Hkv, Sq, L, D)[1:]
    vc = _pack_codes(np.ones((B, Hkv, L, D), int))
    vs = np.full((B, Hkv, L), _h(1.0), np.uint16)
    q = f32_to_bf16_bits((3 * rng.standard_normal((B, Hq, Sq, D))).astype(np.float32))
    for causal in (False, True):
        o, _ = attention(q, kc, ks, vc, vs, L, 0.5, causal)
        assert np.max(np.abs(o - 1.0)) < 1e-14


def test_kv_permutation_invariance():
    q, kc, ks, vc, vs = _rand_case(13, 2, 4, 2, 3, 40, 16)
    perm = np.random.default_rng(0).permutation(40)
    o1, l1 = attention(q, kc, ks, vc, vs, 40, 0.25)
    o2, l2 = attention(q, kc[:, :, perm], ks[:, :, perm], vc[:, :, perm], vs[:, :, perm], 40, 0.25)
    assert np.max(np.abs(o1 - o2)) < 1e-13 and np.max(np.abs(l1 - l2)) < 1e-13


@pytest.mark.parametrize("nparts", [1, 2, 3, 7, 37])
def test_split_merge_invariance(nparts):
    L = 37
    q, kc, ks, vc, vs = _rand_case(14, 2, 4, 2, 2, L, 16)
    o, l = attention(q, kc, ks, vc, vs, L, 0.3)
    edges = np.linspace(0, L, nparts + 1).round().astype(int)
    parts = [attention_partial(q, kc, ks, vc, vs, a, b, 0.3) for a, b in zip(edges[:-1], edges[1:])]
    om, lm = lse_merge(parts)
    assert np.max(np.abs(o - om)) < 1e-13 and np.max(np.abs(l - lm)) < 1e-13


def test_gqa_equals_mha_with_repeated_kv():
    q, kc, ks, vc, vs = _rand_case(15, 2, 8, 2, 3, 21, 16)
    o1, l1 = attention(q, kc, ks, vc, vs, 21, 0.2, causal=True)
    rep = lambda a: np.repeat(a, 4, axis=1)
    o2, l2 = attention(q, rep(kc), rep(ks), rep(vc), rep(vs), 21, 0.2, causal=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_kv_len_prefix_only():
    # rows at and beyond kv_len never matter
    q, kc, ks, vc, vs = _rand_case(16, 1, 2, 2, 2, 10, 8, C=16)
    o1, _ = attention(q, kc, ks, vc, vs, 10, 0.3)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, :, 10:] ^= 0x5A
    vc2[:, :, 10:] ^= 0xA5
    o2, _ = attention(q, kc2, ks, vc2, vs, 10, 0.3)
    assert np.array_equal(o1, o2)


def test_row_subset_matches_full_rows():
    q, kc, ks, vc, vs = _rand_case(17, 1, 4, 2, 40, 50, 8)
    rows = [0, 1, 17, 39]
    for causal in (False, True):
        o1, l1 = attention(q, kc, ks, vc, vs, 50, 0.3, causal)
        o2, l2 = attention(q, kc, ks, vc, vs, 50, 0.3, causal, rows=rows)
        assert np.array_equal(o1[:, :, rows], o2[:, :, rows])
        assert np.array_equal(l1[:, :, rows], l2[:, :, rows])
        assert np.all(np.isnan(np.delete(o2, rows, axis=2)))

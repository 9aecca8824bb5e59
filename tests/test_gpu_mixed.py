"""GPU parity of per-head bit widths (a layer's KV heads split between a
2- or 3-bit cache and a 4-bit cache): quantize-append through a head map
byte for byte against the oracle quantizer, the mixed decode against the
fp64 oracle of each width on its heads, the identity map against the plain
decode bit for bit, and rows of other heads left untouched."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_flashattention_amd as qkv
from gpu_helpers import DEV, assert_close, compare, q_to_dev
from qkv_inputs import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _heads(ids):
    return torch.tensor(ids, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("D", [64, 128])
def test_quantize_through_head_map(bits, D):
    rng = np.random.default_rng(bits + D)
    B, Hkv, T, C, pos = 2, 8, 37, 50, 9
    k = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    ids = [6, 1, 3]
    rb = D * bits // 8
    cache = qkv.KVCache(*(torch.full(sh, f, dtype=dt, device=DEV) for sh, f, dt in (
        ((B, 3, C, rb), 0xA5, torch.uint8), ((B, 3, C), 1.5, torch.float16),
        ((B, 3, C, rb), 0x5A, torch.uint8), ((B, 3, C), -2.5, torch.float16))))
    qkv.quantize_append_kv_heads(_dev(k), _dev(v), cache, _heads(ids), pos, bits=bits)
    torch.cuda.synchronize()
    for src, codes, scales, fc in ((k, cache.k_codes, cache.k_scales, 0xA5), (v, cache.v_codes, cache.v_scales, 0x5A)):
        rc, rs = oracle.quantize_rows_bits(src[:, ids], bits)
        c = codes.cpu().numpy()
        s = scales.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(c[:, :, pos:pos + T], rc) and np.array_equal(s[:, :, pos:pos + T], rs)
        assert np.all(c[:, :, :pos] == fc) and np.all(c[:, :, pos + T:] == fc)


def _layer(seed, B, Hq, Hkv, Sq, L, D):
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, Sq, D)).astype(np.float32))
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    k[:, :, :, rng.choice(D, 2, replace=False)] *= 8.0
    return q, k, v


def _oracle_part(q, k, v, ids, bits, L, scale, G):
    qi = [h * G + i for h in ids for i in range(G)]
    kc, ks = oracle.quantize_rows_bits(k[:, ids], bits)
    vc, vs = oracle.quantize_rows_bits(v[:, ids], bits)
    o, l = oracle.attention_bits(q[:, qi], kc, ks, vc, vs, L, scale, bits)
    return qi, o, l


CASES = [
    # B, Hq, Hkv, Sq, L, D, low-bit heads, low bits, num_splits
    (2, 32, 8, 1, 1000, 128, [1, 4, 6], 2, 0),
    (1, 16, 8, 2, 777, 128, [7, 0], 3, 3),
    (2, 8, 4, 1, 300, 64, [2], 2, 0),
    (1, 64, 8, 1, 4097, 128, [0, 1, 2, 3], 2, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_mixed_decode_matches_oracle(case):
    B, Hq, Hkv, Sq, L, D, lo_ids, lo_bits, ns = case
    G = Hq // Hkv
    q, k, v = _layer(sum(case[:6]), B, Hq, Hkv, Sq, L, D)
    hi_ids = [h for h in range(Hkv) if h not in lo_ids]
    scale = float(np.float32(1 / np.sqrt(D)))
    parts, want_o, want_l = [], np.full((B, Hq, Sq, D), np.nan), np.full((B, Hq, Sq), np.nan)
    for ids, bits in ((lo_ids, lo_bits), (hi_ids, 4)):
        cache = qkv.KVCache.empty(B, len(ids), L, D, device=DEV, bits=bits)
        qkv.quantize_append_kv_heads(_dev(k), _dev(v), cache, _heads(ids), 0, bits=bits)
        parts.append((cache, _heads(ids), bits))
        qi, o, l = _oracle_part(q, k, v, ids, bits, L, scale, G)
        want_o[:, qi], want_l[:, qi] = o, l
    out = torch.full((B, Hq, Sq, D), float("nan"), device=DEV)
    out, lse = qkv.decode_mixed(q_to_dev(q), parts, Hkv, L, softmax_scale=scale, num_splits=ns, return_lse=True,
                                out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "a query row was not written"
    assert_close(out, want_o, f"mixed {case}")
    assert compare(lse, want_l)[0] < 1e-3


def test_identity_head_map_is_plain_decode():
    B, Hq, Hkv, L, D = 2, 32, 8, 2000, 128
    q, k, v = _layer(3, B, Hq, Hkv, 1, L, D)
    cache = qkv.KVCache.empty(B, Hkv, L, D, device=DEV)
    qkv.quantize_append_kv_heads(_dev(k), _dev(v), cache, _heads(list(range(Hkv))), 0)
    plain = qkv.KVCache.empty(B, Hkv, L, D, device=DEV)
    qkv.quantize_append_kv(_dev(k), _dev(v), plain, 0)
    out = torch.empty((B, Hq, 1, D), device=DEV)
    qkv.decode_heads(q_to_dev(q), cache, _heads(list(range(Hkv))), Hkv, L, out, num_splits=3)
    ref = qkv.decode(q_to_dev(q), plain, L, num_splits=3)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(cache.tensors(), plain.tensors()))
    assert torch.equal(out, ref)


def test_other_heads_untouched():
    B, Hq, Hkv, L, D = 1, 16, 8, 500, 128
    q, k, v = _layer(4, B, Hq, Hkv, 1, L, D)
    ids = [5, 2]
    cache = qkv.KVCache.empty(B, 2, L, D, device=DEV, bits=2)
    qkv.quantize_append_kv_heads(_dev(k), _dev(v), cache, _heads(ids), 0, bits=2)
    out = torch.full((B, Hq, 1, D), 7.0, device=DEV)
    lse = torch.full((B, Hq, 1), 7.0, device=DEV)
    qkv.decode_heads(q_to_dev(q), cache, _heads(ids), Hkv, L, out, lse=lse, bits=2)
    torch.cuda.synchronize()
    G = Hq // Hkv
    mine = [h * G + i for h in ids for i in range(G)]
    others = [h for h in range(Hq) if h not in mine]
    assert torch.all(out[:, others] == 7.0) and torch.all(lse[:, others] == 7.0)
    qi, o, _ = _oracle_part(q, k, v, ids, 2, L, float(np.float32(1 / np.sqrt(D))), G)
    assert_close(out[:, qi], o, "head subset")


PREFILL_CASES = [
    # B, Hq, Hkv, Sq, L, D, low-bit heads, low bits, causal
    (1, 32, 8, 300, 300, 128, [1, 4, 6], 2, True),
    (2, 8, 4, 197, 197, 64, [2], 3, False),
    (1, 16, 8, 100, 500, 128, [7, 0], 2, True),      # Sq < kv_len
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[str(c) for c in PREFILL_CASES])
def test_mixed_prefill_matches_oracle(case):
    B, Hq, Hkv, Sq, L, D, lo_ids, lo_bits, causal = case
    G = Hq // Hkv
    q, k, v = _layer(sum(case[:6]), B, Hq, Hkv, Sq, L, D)
    hi_ids = [h for h in range(Hkv) if h not in lo_ids]
    scale = float(np.float32(1 / np.sqrt(D)))
    parts, want_o, want_l = [], np.full((B, Hq, Sq, D), np.nan), np.full((B, Hq, Sq), np.nan)
    for ids, bits in ((lo_ids, lo_bits), (hi_ids, 4)):
        cache = qkv.KVCache.empty(B, len(ids), L, D, device=DEV, bits=bits)
        qkv.quantize_append_kv_heads(_dev(k), _dev(v), cache, _heads(ids), 0, bits=bits)
        parts.append((cache, _heads(ids), bits))
        qi = [h * G + i for h in ids for i in range(G)]
        kc, ks = oracle.quantize_rows_bits(k[:, ids], bits)
        vc, vs = oracle.quantize_rows_bits(v[:, ids], bits)
        want_o[:, qi], want_l[:, qi] = oracle.attention_bits(q[:, qi], kc, ks, vc, vs, L, scale, bits, causal=causal)
    out = torch.full((B, Hq, Sq, D), float("nan"), device=DEV)
    out, lse = qkv.prefill_mixed(q_to_dev(q), parts, Hkv, L, causal, softmax_scale=scale, return_lse=True, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "a query row was not written"
    assert_close(out, want_o, f"mixed prefill {case}")
    assert compare(lse, want_l)[0] < 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_identity_head_map_is_plain_prefill(causal):
    B, Hq, Hkv, Sq, L, D = 1, 16, 4, 250, 250, 128
    q, k, v = _layer(5 + causal, B, Hq, Hkv, Sq, L, D)
    plain = qkv.KVCache.empty(B, Hkv, L, D, device=DEV)
    qkv.quantize_append_kv(_dev(k), _dev(v), plain, 0)
    out = torch.empty((B, Hq, Sq, D), device=DEV)
    lse = torch.empty((B, Hq, Sq), device=DEV)
    qkv.prefill_heads(q_to_dev(q), plain, _heads(list(range(Hkv))), Hkv, L, causal, out, lse=lse)
    ro, rl = qkv.prefill(q_to_dev(q), plain, L, causal, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ro) and torch.equal(lse, rl)


def test_prefill_other_heads_untouched():
    B, Hq, Hkv, Sq, L, D = 1, 16, 8, 130, 130, 64
    q, k, v = _layer(6, B, Hq, Hkv, Sq, L, D)
    ids = [5, 2]
    cache = qkv.KVCache.empty(B, 2, L, D, device=DEV, bits=3)
    qkv.quantize_append_kv_heads(_dev(k), _dev(v), cache, _heads(ids), 0, bits=3)
    out = torch.full((B, Hq, Sq, D), 7.0, device=DEV)
    lse = torch.full((B, Hq, Sq), 7.0, device=DEV)
    qkv.prefill_heads(q_to_dev(q), cache, _heads(ids), Hkv, L, True, out, lse=lse, bits=3)
    torch.cuda.synchronize()
    G = Hq // Hkv
    mine = [h * G + i for h in ids for i in range(G)]
    others = [h for h in range(Hq) if h not in mine]
    assert torch.all(out[:, others] == 7.0) and torch.all(lse[:, others] == 7.0)
    kc, ks = oracle.quantize_rows_bits(k[:, ids], 3)
    vc, vs = oracle.quantize_rows_bits(v[:, ids], 3)
    o, _ = oracle.attention_bits(q[:, mine], kc, ks, vc, vs, L, float(np.float32(1 / np.sqrt(D))), 3, causal=True)
    assert_close(out[:, mine], o, "head subset")

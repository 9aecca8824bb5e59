"""GPU parity of 2- and 3-bit rows: quantize-append byte for byte against the
oracle quantizer, decode against the fp64 oracle, and decode of b-bit rows
against the int4 decode of the same codes (a 2- or 3-bit code is an int4 code
under the same scale): equal up to fp32 rounding, since each width feeds the
matrix units its codes plus a width-specific bias that fp32 sums remove)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_flashattention_amd as qkv
from gpu_helpers import DEV, assert_close, compare, q_to_dev
from qkv_inputs import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _scales_np(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _rows(rng, B, H, T, D):
    x = rng.standard_normal((B, H, T, D)).astype(np.float32)
    x[0, 0] *= np.float32(2.0) ** rng.integers(-25, 10, size=(T, 1)).astype(np.float32)   # wide magnitudes
    x[0, -1, ::4] = 0.0                                                                      # zero rows
    ties = (rng.integers(-3, 3, size=(T, D)) + 0.5).astype(np.float32)
    ties[:, 0] = 3.0
    x[-1, 0] = ties * np.float32(0.25)                                                       # exact ties (3-bit)
    return x


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T,C,pos", [(1, 5, 4), (37, 50, 13), (300, 310, 0)])
def test_quantize_append_matches_oracle(bits, D, T, C, pos):
    rng = np.random.default_rng(bits * 1000 + D + T)
    k, v = _rows(rng, 2, 3, T, D), _rows(rng, 2, 3, T, D)
    rb = D * bits // 8
    cache = qkv.KVCache(*(torch.full(sh, f, dtype=dt, device=DEV) for sh, f, dt in (
        ((2, 3, C, rb), 0xA5, torch.uint8), ((2, 3, C), 1.5, torch.float16),
        ((2, 3, C, rb), 0x5A, torch.uint8), ((2, 3, C), -2.5, torch.float16))))
    qkv.quantize_append_kv(torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV), cache, pos, bits=bits)
    torch.cuda.synchronize()
    for src, codes, scales, fc in ((k, cache.k_codes, cache.k_scales, 0xA5), (v, cache.v_codes, cache.v_scales, 0x5A)):
        rc, rs = oracle.quantize_rows_bits(src, bits)
        c, s = codes.cpu().numpy(), _scales_np(scales)
        assert np.array_equal(c[:, :, pos:pos + T], rc) and np.array_equal(s[:, :, pos:pos + T], rs)
        assert np.all(c[:, :, :pos] == fc) and np.all(c[:, :, pos + T:] == fc)


def _lowbit_case(seed, B, Hq, Hkv, Sq, L, C, D, bits):
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, Sq, D)).astype(np.float32))
    out = []
    for scale in (1.0, 1.5):
        x = (rng.standard_normal((B, Hkv, C, D)) * scale).astype(np.float32)
        ch = rng.choice(D, size=2, replace=False)
        x[:, :, :, ch] *= 8.0                            # outlier channels
        out += list(oracle.quantize_rows_bits(x, bits))
    return q, out


def _to_dev(arrs):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    h = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).to(DEV)
    return qkv.KVCache(t(arrs[0]), h(arrs[1]), t(arrs[2]), h(arrs[3]))


def _as_int4(codes, D, bits):
    c = oracle.unpack_bits(codes, D, bits).astype(np.int64) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


CASES = [
    # B, Hq, Hkv, Sq, L, C, D, num_splits
    (2, 8, 2, 1, 1000, 1024, 128, 0),
    (1, 64, 8, 1, 4097, 4100, 128, 0),
    (2, 32, 8, 2, 777, 800, 128, 3),
    (1, 8, 2, 5, 129, 129, 64, 0),       # 20 rows per group: two 16-row blocks
    (1, 4, 1, 16, 300, 300, 128, 0),     # 64 rows per group
    (1, 8, 8, 1, 33, 40, 64, 1),
    (3, 12, 4, 3, 2049, 2100, 128, 5),
]


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_decode_bits_matches_oracle_and_int4(case, bits):
    B, Hq, Hkv, Sq, L, C, D, ns = case
    q, (kc, ks, vc, vs) = _lowbit_case(sum(case) + bits, B, Hq, Hkv, Sq, L, C, D, bits)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse = qkv.decode(q_to_dev(q), _to_dev((kc, ks, vc, vs)), L, softmax_scale=scale, num_splits=ns,
                          return_lse=True, bits=bits)
    o4, l4 = qkv.decode(q_to_dev(q), _to_dev((_as_int4(kc, D, bits), ks, _as_int4(vc, D, bits), vs)), L,
                        softmax_scale=scale, num_splits=ns, return_lse=True)
    torch.cuda.synchronize()
    # the same codes through the int4 kernel: equal up to fp32 rounding (the
    # widths convert codes with different biases, removed in fp32 sums)
    assert float((out - o4).abs().max()) <= 1e-3, f"differs from the int4 decode: {float((out - o4).abs().max())}"
    assert float((lse - l4).abs().max()) <= 1e-3
    ro, rl = oracle.attention_bits(q, kc, ks, vc, vs, L, scale, bits)
    assert_close(out, ro, f"bits={bits} {case}")
    assert compare(lse, rl)[0] < 1e-3


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("L", [1, 31, 32, 33, 65, 197])
def test_decode_bits_length_edges(bits, L):
    q, arrs = _lowbit_case(L + bits, 2, 4, 2, 1, L, L + 3, 64, bits)
    out = qkv.decode(q_to_dev(q), _to_dev(arrs), L, softmax_scale=0.125, bits=bits)
    torch.cuda.synchronize()
    ro, _ = oracle.attention_bits(q, *arrs, L, 0.125, bits)
    assert_close(out, ro, f"bits={bits} L={L}")


PREFILL_CASES = [
    # B, Hq, Hkv, Sq, L, C, D, causal
    (1, 8, 2, 300, 300, 320, 128, True),
    (2, 4, 4, 197, 197, 197, 64, False),
    (1, 8, 2, 100, 700, 700, 128, True),      # Sq < kv_len: bottom-right aligned
    (1, 4, 1, 513, 600, 640, 64, True),
    (1, 4, 2, 70, 1000, 1024, 128, False),
]


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("case", PREFILL_CASES, ids=[str(c) for c in PREFILL_CASES])
def test_prefill_bits_matches_oracle(case, bits):
    B, Hq, Hkv, Sq, L, C, D, causal = case
    # outlier channels in K and V (V values up to ~40: early causal rows see
    # few keys, so P~ takes its hi/lo form where the V scales are large)
    q, (kc, ks, vc, vs) = _lowbit_case(sum(case) + bits, B, Hq, Hkv, Sq, L, C, D, bits)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out = torch.full((B, Hq, Sq, D), float("nan"), device=DEV)
    out, lse = qkv.prefill(q_to_dev(q), _to_dev((kc, ks, vc, vs)), L, causal, softmax_scale=scale,
                           return_lse=True, out=out, bits=bits)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_bits(q, kc, ks, vc, vs, L, scale, bits, causal=causal)
    assert_close(out, ro, f"prefill bits={bits} {case}")
    assert compare(lse, rl)[0] < 1e-3


@pytest.mark.parametrize("bits", [2, 3])
def test_prefill_bits_causal_16k_sampled(bits):
    """The causal prefill workload's shape (32/8 heads, D 128, 16384 tokens) over
    b-bit rows, checked on sampled query rows of every head."""
    B, Hq, Hkv, L, D = 1, 32, 8, 16384, 128
    rng = np.random.default_rng(40 + bits)
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, L, D)).astype(np.float32))
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    cache = qkv.KVCache.empty(B, Hkv, L, D, device=DEV, bits=bits)
    qkv.quantize_append_kv(torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV), cache, 0, bits=bits)
    out = qkv.prefill(q_to_dev(q), cache, L, True, bits=bits)
    torch.cuda.synchronize()
    kc, ks = oracle.quantize_rows_bits(k, bits)
    vc, vs = oracle.quantize_rows_bits(v, bits)
    rows = np.array([0, 1, 63, 64, 4095, 8191, 12000, L - 1])
    scale = float(np.float32(1.0 / np.sqrt(D)))
    errs = []
    for r in rows:
        qr = q[:, :, r:r + 1]
        ro, _ = oracle.attention_bits(qr, kc, ks, vc, vs, r + 1, scale, bits)   # row r sees keys [0, r]
        errs.append(np.abs(out[:, :, r:r + 1].cpu().double().numpy() - ro))
    e = np.concatenate([x.ravel() for x in errs])
    assert e.max() <= 4e-3 and e.mean() <= 4e-4, (e.max(), e.mean())

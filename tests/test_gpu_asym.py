"""GPU parity of asymmetric group-wise int4 rows: quantize-append byte for byte
(codes in the cache's row orders, and parameter words) against the oracle
quantizer, decode against the fp64 oracle over caches with garbage past
kv_len, and decode of symmetric int4 rows embedded as asymmetric rows (zero
point 8) against the symmetric decode of the same rows."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_flashattention_amd as qkv
from gpu_helpers import DEV, assert_close, compare, q_to_dev, random_case
from qkv_inputs import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _params(scales, zeros):
    """Parameter words: fp16 scale bits | zero point << 16 (as int32)."""
    return (scales.astype(np.uint32) | (zeros.astype(np.uint32) << 16)).view(np.int32)


def _rows(rng, B, H, T, D, group):
    x = rng.standard_normal((B, H, T, D)).astype(np.float32)
    x[0, 0] *= np.float32(2.0) ** rng.integers(-25, 10, size=(T, 1)).astype(np.float32)   # wide magnitudes
    x[0, -1, ::4] = 0.0                                                                      # zero rows
    x[-1, 0, :, :group] = np.abs(x[-1, 0, :, :group]) + 0.5                                  # all-positive groups
    x[-1, -1, :, -group:] = -np.abs(x[-1, -1, :, -group:]) - 0.25                            # all-negative groups
    x[0, 0, ::3, group:2 * group if 2 * group <= D else group] = 0.0                          # zero groups
    s = np.float16(0.125)                                                                      # exact ties
    k = (rng.integers(-5, 10, size=(T, D)) + 0.5).astype(np.float32)
    k[:, ::group] = -5.0
    k[:, 1::group] = 10.0
    x[-1, 1 % H] = k * np.float32(s)
    return x


GROUPS = [(64, 32), (64, 64), (128, 32), (128, 64), (128, 128)]


@pytest.mark.parametrize("D,group", GROUPS)
@pytest.mark.parametrize("T,C,pos", [(1, 5, 4), (37, 50, 13), (300, 310, 0)])
def test_quantize_append_matches_oracle(D, group, T, C, pos):
    rng = np.random.default_rng(D + group + T)
    B, H = 2, 3
    k, v = _rows(rng, B, H, T, D, group), _rows(rng, B, H, T, D, group)
    cache = qkv.AsymKVCache(
        torch.full((B, H, C, D // 2), 0xA5, dtype=torch.uint8, device=DEV),
        torch.full((B, H, C, D // group), 0x1234, dtype=torch.int32, device=DEV),
        torch.full((B, H, C, D // 2), 0x5A, dtype=torch.uint8, device=DEV),
        torch.full((B, H, C, D // group), -7, dtype=torch.int32, device=DEV), group)
    qkv.quantize_append_kv_asym(torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV), cache, pos)
    torch.cuda.synchronize()
    for src, codes, params, fc, fp in ((k, cache.k_codes, cache.k_params, 0xA5, 0x1234),
                                       (v, cache.v_codes, cache.v_params, 0x5A, -7)):
        rc, rs, rz = oracle.quantize_rows_asym(src, group)
        rc = oracle.to_cache_order(rc, "k" if fc == 0xA5 else "v")
        c, p = codes.cpu().numpy(), params.cpu().numpy()
        assert np.array_equal(c[:, :, pos:pos + T], rc), "codes differ"
        assert np.array_equal(p[:, :, pos:pos + T], _params(rs, rz)), "scale / zero point words differ"
        assert np.all(c[:, :, :pos] == fc) and np.all(c[:, :, pos + T:] == fc)
        assert np.all(p[:, :, :pos] == fp) and np.all(p[:, :, pos + T:] == fp)


def _asym_case(seed, B, Hq, Hkv, Sq, L, C, D, group):
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, Sq, D)).astype(np.float32))
    out = []
    for shift in (0.0, 0.7):
        x = (rng.standard_normal((B, Hkv, C, D)) + shift).astype(np.float32)   # V off centre: zero points matter
        ch = rng.choice(D, size=2, replace=False)
        x[:, :, :, ch] *= 8.0                                                  # outlier channels
        c, s, z = oracle.quantize_rows_asym(x, group)
        c[:, :, L:] = rng.integers(0, 256, size=c[:, :, L:].shape, dtype=np.uint8)   # garbage past kv_len
        s[:, :, L:] = rng.integers(0, 0x7800, size=s[:, :, L:].shape, dtype=np.uint16)
        z[:, :, L:] = rng.integers(0, 16, size=z[:, :, L:].shape, dtype=np.uint8)
        out += [c, s, z]
    return q, out


def _to_dev(arrs, group):
    """Oracle rows (element order) -> a device cache (the cache's row orders)."""
    kc, ks, kz, vc, vs, vz = arrs
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return qkv.AsymKVCache(t(oracle.to_cache_order(kc, "k")), t(_params(ks, kz)),
                           t(oracle.to_cache_order(vc, "v")), t(_params(vs, vz)), group)


CASES = [
    # B, Hq, Hkv, Sq, L, C, D, group, num_splits
    (2, 8, 2, 1, 1000, 1024, 128, 32, 0),
    (1, 64, 8, 1, 4097, 4100, 128, 64, 0),
    (2, 32, 8, 2, 777, 800, 128, 128, 3),
    (1, 8, 2, 5, 129, 129, 64, 32, 0),       # 20 rows per group: two 16-row blocks
    (1, 4, 1, 16, 300, 300, 128, 32, 0),     # 64 rows per group
    (1, 8, 8, 1, 33, 40, 64, 64, 1),
    (3, 12, 4, 3, 2049, 2100, 128, 64, 5),
    (1, 2, 2, 1, 1, 8, 64, 32, 0),           # a single row
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_decode_asym_matches_oracle(case):
    B, Hq, Hkv, Sq, L, C, D, group, ns = case
    q, arrs = _asym_case(sum(case), B, Hq, Hkv, Sq, L, C, D, group)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out = torch.full((B, Hq, Sq, D), float("nan"), device=DEV)
    out, lse = qkv.decode_asym(q_to_dev(q), _to_dev(arrs, group), L, softmax_scale=scale, num_splits=ns,
                               return_lse=True, out=out)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_asym(q, *arrs, L, scale, group)
    assert_close(out, ro, f"asym {case}")
    assert compare(lse, rl)[0] < 1e-3


def test_decode_asym_split_counts_agree_and_are_deterministic():
    case = (2, 32, 8, 1, 3000, 3000, 128, 32)
    q, arrs = _asym_case(7, *case)
    cache = _to_dev(arrs, 32)
    qd = q_to_dev(q)
    ro, _ = oracle.attention_asym(q, *arrs, 3000, float(np.float32(1 / np.sqrt(128))), 32)
    outs = {}
    for ns in (1, 2, 7, 0):
        a = qkv.decode_asym(qd, cache, 3000, num_splits=ns)
        b = qkv.decode_asym(qd, cache, 3000, num_splits=ns)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"run-to-run difference at ns={ns}"
        assert_close(a, ro, f"ns={ns}")
        outs[ns] = a
    for ns, a in outs.items():
        assert float((a - outs[1]).abs().max()) < 1e-3   # fp32 merge order only


@pytest.mark.parametrize("D", [64, 128])
def test_symmetric_rows_embedded(D):
    """Symmetric int4 rows as asymmetric rows (codes + 8, zero point 8, one
    group per row): the same values, so the asymmetric decode agrees with the
    symmetric decode up to fp32 rounding (the two convert codes with
    different biases)."""
    B, Hq, Hkv, L = 2, 16, 4, 1500
    q, kc, ks, vc, vs = random_case(5, B, Hq, Hkv, 1, L, D)
    emb = lambda c: (c.astype(np.int64) ^ 0x88).astype(np.uint8)   # flip each nibble's top bit: c + 8
    z = np.full((B, Hkv, L, 1), 8, np.uint8)
    cache = qkv.AsymKVCache(*(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (
        oracle.to_cache_order(emb(kc), "k"), _params(ks[..., None], z),
        oracle.to_cache_order(emb(vc), "v"), _params(vs[..., None], z))), group=D)
    sym = qkv.KVCache(*(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (
        kc, ks.view(np.float16), vc, vs.view(np.float16))))
    oa = qkv.decode_asym(q_to_dev(q), cache, L)
    os_ = qkv.decode(q_to_dev(q), sym, L)
    torch.cuda.synchronize()
    d = (oa - os_).abs()
    assert float(d.max()) < 2e-4 and float(d.mean()) < 2e-5
    ro, _ = oracle.attention(q, kc, ks, vc, vs, L, float(np.float32(1 / np.sqrt(D))))
    assert_close(oa, ro, "embedded symmetric rows")


def test_quantize_then_decode_end_to_end():
    """Quantize on the GPU, then decode: equals the oracle over the oracle's own quantization."""
    rng = np.random.default_rng(21)
    B, Hq, Hkv, L, D, group = 2, 16, 4, 900, 128, 64
    k = (rng.standard_normal((B, Hkv, L, D)) + 0.3).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, 1, D)).astype(np.float32))
    cache = qkv.AsymKVCache.empty(B, Hkv, L, D, group, device=DEV)
    qkv.quantize_append_kv_asym(torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV), cache, 0)
    out = qkv.decode_asym(q_to_dev(q), cache, L)
    torch.cuda.synchronize()
    kq = oracle.quantize_rows_asym(k, group)
    vq = oracle.quantize_rows_asym(v, group)
    ro, _ = oracle.attention_asym(q, *kq, *vq, L, float(np.float32(1 / np.sqrt(D))), group)
    assert_close(out, ro, "quantize + decode")


def _prefill_case(seed, B, Hq, Hkv, Sq, L, C, D, group):
    """K and V with outlier channels and an offset (zero points matter); with
    few visible keys (early causal rows) P~ takes its hi/lo form on tiles
    whose V group scales are large."""
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, Sq, D)).astype(np.float32))
    out = []
    for shift in (0.4, 0.7):
        x = (rng.standard_normal((B, Hkv, C, D)) + shift).astype(np.float32)
        x[:, :, :, rng.choice(D, size=2, replace=False)] *= 8.0
        c, s, z = oracle.quantize_rows_asym(x, group)
        c[:, :, L:] = rng.integers(0, 256, size=c[:, :, L:].shape, dtype=np.uint8)   # garbage past kv_len
        s[:, :, L:] = rng.integers(0, 0x7800, size=s[:, :, L:].shape, dtype=np.uint16)
        z[:, :, L:] = rng.integers(0, 16, size=z[:, :, L:].shape, dtype=np.uint8)
        out += [c, s, z]
    return q, out


PREFILL_CASES = [
    # B, Hq, Hkv, Sq, L, C, D, group, causal
    (1, 8, 2, 300, 300, 320, 128, 32, True),
    (1, 8, 2, 300, 300, 320, 128, 64, True),
    (1, 8, 2, 300, 300, 320, 128, 128, True),
    (2, 4, 4, 197, 197, 197, 64, 32, False),
    (2, 4, 4, 197, 197, 197, 64, 64, False),
    (1, 8, 2, 100, 700, 700, 128, 32, True),     # Sq < kv_len: bottom-right aligned
    (1, 4, 1, 513, 600, 640, 64, 32, True),
    (1, 4, 2, 70, 1000, 1024, 128, 64, False),
    (1, 8, 8, 33, 33, 40, 128, 32, True),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[str(c) for c in PREFILL_CASES])
def test_prefill_asym_matches_oracle(case):
    B, Hq, Hkv, Sq, L, C, D, group, causal = case
    q, arrs = _prefill_case(sum(case), B, Hq, Hkv, Sq, L, C, D, group)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out = torch.full((B, Hq, Sq, D), float("nan"), device=DEV)
    out, lse = qkv.prefill_asym(q_to_dev(q), _to_dev(arrs, group), L, causal, softmax_scale=scale,
                                return_lse=True, out=out)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_asym(q, *arrs, L, scale, group, causal=causal)
    assert_close(out, ro, f"prefill asym {case}")
    assert compare(lse, rl)[0] < 1e-3


@pytest.mark.parametrize("vscale", [0.25, 8.0], ids=["small_v", "large_v"])
@pytest.mark.parametrize("D,group", [(64, 64), (128, 128), (128, 32)])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_symmetric_rows_embedded(D, group, causal, vscale):
    """Symmetric int4 rows as asymmetric rows (codes + 8, zero point 8, the
    row's scale for every group): the same fp16 operands, so with one group
    per row the asymmetric prefill equals the int4 prefill bit for bit; with
    several, the per-group scaling changes only the fp32 rounding order.
    V scales are multiplied by a power of two so that both kernels take the
    same form of P~ on every tile: single fp16 values (scales below both
    kernels' limits) or hi/lo pairs (above both)."""
    B, Hq, Hkv, Sq, L = 1, 8, 2, 200, 260
    q, kc, ks, vc, vs = random_case(9 + D + group, B, Hq, Hkv, Sq, L, D)
    vs = (vs.view(np.float16) * np.float16(vscale)).view(np.uint16)   # exact
    emb = lambda c: (c.astype(np.int64) ^ 0x88).astype(np.uint8)
    ng = D // group
    z = np.full((B, Hkv, L, ng), 8, np.uint8)
    rep = lambda s_: np.repeat(s_[..., None], ng, axis=-1)
    cache = qkv.AsymKVCache(*(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (
        oracle.to_cache_order(emb(kc), "k"), _params(rep(ks), z),
        oracle.to_cache_order(emb(vc), "v"), _params(rep(vs), z))), group=group)
    sym = qkv.KVCache(*(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (
        kc, ks.view(np.float16), vc, vs.view(np.float16))))
    oa = qkv.prefill_asym(q_to_dev(q), cache, L, causal)
    os_ = qkv.prefill(q_to_dev(q), sym, L, causal)
    torch.cuda.synchronize()
    if ng == 1:
        assert torch.equal(oa, os_)
    else:   # fp32 summation order only: differences scale with the V magnitudes
        d = (oa - os_).abs()
        assert float(d.max()) < 1e-4 * max(vscale, 1.0) and float(d.mean()) < 1e-5 * max(vscale, 1.0)
    ro, _ = oracle.attention(q, kc, ks, vc, vs, L, float(np.float32(1 / np.sqrt(D))), causal=causal)
    assert_close(oa, ro, "embedded symmetric rows")


@pytest.mark.parametrize("group", [32, 128])
def test_prefill_asym_causal_16k_sampled(group):
    """The causal prefill workload's shape (32/8 heads, D 128, 16384 tokens)
    over asymmetric rows quantized on the GPU, checked on sampled query rows
    of every head."""
    B, Hq, Hkv, L, D = 1, 32, 8, 16384, 128
    rng = np.random.default_rng(60 + group)
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, L, D)).astype(np.float32))
    k = (rng.standard_normal((B, Hkv, L, D)) + 0.3).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    cache = qkv.AsymKVCache.empty(B, Hkv, L, D, group, device=DEV)
    qkv.quantize_append_kv_asym(torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV), cache, 0)
    out = qkv.prefill_asym(q_to_dev(q), cache, L, True)
    torch.cuda.synchronize()
    kq = oracle.quantize_rows_asym(k, group)
    vq = oracle.quantize_rows_asym(v, group)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    errs = []
    for r in [0, 1, 63, 64, 4095, 8191, 12000, L - 1]:
        ro, _ = oracle.attention_asym(q[:, :, r:r + 1], *kq, *vq, r + 1, scale, group)   # row r sees keys [0, r]
        errs.append(np.abs(out[:, :, r:r + 1].cpu().double().numpy() - ro))
    e = np.concatenate([x.ravel() for x in errs])
    assert e.max() <= 4e-3 and e.mean() <= 4e-4, (e.max(), e.mean())


@pytest.mark.parametrize("D,group", [(64, 32), (128, 64), (128, 32)])
@pytest.mark.parametrize("L,Sq,causal", [(1, 1, True), (1, 1, False), (63, 63, True), (64, 64, True),
                                         (65, 65, True), (129, 129, False), (200, 1, True)])
def test_prefill_asym_length_edges(D, group, L, Sq, causal):
    """A single key, lengths at and around the 64-token tile, and one query row
    against a longer cache (causal: it sees every key)."""
    B, Hq, Hkv = 1, 4, 2
    q, arrs = _prefill_case(L * 7 + Sq + D + group + causal, B, Hq, Hkv, Sq, L, L + 5, D, group)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out = qkv.prefill_asym(q_to_dev(q), _to_dev(arrs, group), L, causal, softmax_scale=scale)
    torch.cuda.synchronize()
    ro, _ = oracle.attention_asym(q, *arrs, L, scale, group, causal=causal)
    assert_close(out, ro, f"asym prefill L={L} Sq={Sq} causal={causal} D={D} g={group}")

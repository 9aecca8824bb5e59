"""GPU parity where one fp16 rounding of P~ = p s_V would not hold the
tolerance, and at the edges of the fp16 operand range.

* V rows with channel outliers (a few channels x8, the structure
  TurboAttention arXiv 2412.08585 §3.1 describes) under concentrated
  attention: a handful of keys, early causal rows, one dominant key.  With
  |v| up to ~60 a single rounding of P~ errs by up to ~60 * 2^-11, past the
  tolerance, so these cases fail unless the kernels take P~ as an fp16 hi/lo
  pair where V scales are large.  Every decode row layout is covered: the packed softmax (at most 4
  query rows), duplicated rows (5-8), and the multi-block kernels (9-64),
  for int4, 2- and 3-bit and asymmetric rows, the paged cache and the fused
  append.
* V scales close to the fp16 maximum (row absmax up to 7 * 65504): the
  prefill's lazy rescale must keep p s_V finite.
* Query elements of magnitude 65536 and more (past fp16 range), with a
  softmax scale that brings the scores back to order one.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_flashattention_amd as qkv
from gpu_helpers import DEV, assert_close, compare, q_to_dev
from qkv_inputs import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

VGAIN = 2.5   # V ~ N(0, 6.25) with x8 outlier channels: |v| up to ~60


def _raw(rng, B, Hq, Hkv, Sq, C, D, vgain=VGAIN, dominant=None):
    """bf16 query bits and fp32 K, V rows; two outlier channels (x8) per tensor.
    dominant = (t, gap): key t of every head gets q's direction scaled so that
    its score leads the others by about `gap` (natural log units)."""
    q = rng.standard_normal((B, Hq, Sq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, C, D)).astype(np.float32)
    v = (rng.standard_normal((B, Hkv, C, D)) * vgain).astype(np.float32)
    for t in (k, v):
        t[..., rng.choice(D, size=2, replace=False)] *= np.float32(8.0)
    if dominant is not None:
        t, gap = dominant
        G = Hq // Hkv
        for g in range(Hkv):
            qd = q[:, g * G:(g + 1) * G].mean(axis=(1, 2))            # [B, D]
            nrm = np.linalg.norm(qd, axis=-1, keepdims=True)
            k[:, g, t] = qd / nrm * np.float32(gap * np.sqrt(D) / max(float(nrm.min()), 1e-3))
    return f32_to_bf16_bits(q), k, v


def _sym_dev(kc, ks, vc, vs):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    h = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).to(DEV)
    return qkv.KVCache(t(kc), h(ks), t(vc), h(vs))


def _params(scales, zeros):
    return (scales.astype(np.uint32) | (zeros.astype(np.uint32) << 16)).view(np.int32)


def _asym_dev(arrs, group):
    kc, ks, kz, vc, vs, vz = arrs
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return qkv.AsymKVCache(t(oracle.to_cache_order(kc, "k")), t(_params(ks, kz)),
                           t(oracle.to_cache_order(vc, "v")), t(_params(vs, vz)), group)


def _decode_case(fmt, seed, B, Hq, Hkv, Sq, L, D, dominant=None):
    """Returns (q, device cache, oracle fn(q, L, scale, causal) -> (out, lse), run(qd, cache, L, scale, **kw))."""
    rng = np.random.default_rng(seed)
    q, k, v = _raw(rng, B, Hq, Hkv, Sq, L, D, dominant=dominant)
    if fmt == "int4":
        kc, ks = oracle.quantize_rows(k)
        vc, vs = oracle.quantize_rows(v)
        ref = lambda qq, LL, sc, causal=False: oracle.attention(qq, kc, ks, vc, vs, LL, sc, causal=causal)
        return q, _sym_dev(kc, ks, vc, vs), ref, {}
    if fmt in ("bits2", "bits3"):
        bits = int(fmt[-1])
        kc, ks = oracle.quantize_rows_bits(k, bits)
        vc, vs = oracle.quantize_rows_bits(v, bits)
        ref = lambda qq, LL, sc, causal=False: oracle.attention_bits(qq, kc, ks, vc, vs, LL, sc, bits, causal=causal)
        return q, _sym_dev(kc, ks, vc, vs), ref, {"bits": bits}
    group = int(fmt[4:])   # "asym32", "asym64", "asym128"
    arrs = list(oracle.quantize_rows_asym(k, group)) + list(oracle.quantize_rows_asym(v, group))
    ref = lambda qq, LL, sc, causal=False: oracle.attention_asym(qq, *arrs, LL, sc, group, causal=causal)
    return q, _asym_dev(arrs, group), ref, {"group": group}


def _decode(fmt, qd, cache, L, scale, ns=0):
    if fmt.startswith("asym"):
        return qkv.decode_asym(qd, cache, L, softmax_scale=scale, num_splits=ns, return_lse=True)
    return qkv.decode(qd, cache, L, softmax_scale=scale, num_splits=ns, return_lse=True,
                      bits=int(fmt[-1]) if fmt.startswith("bits") else 4)


def _prefill(fmt, qd, cache, L, causal, scale):
    if fmt.startswith("asym"):
        return qkv.prefill_asym(qd, cache, L, causal, softmax_scale=scale, return_lse=True)
    return qkv.prefill(qd, cache, L, causal, softmax_scale=scale, return_lse=True,
                       bits=int(fmt[-1]) if fmt.startswith("bits") else 4)


# (G, Sq) -> query rows per group R = G * Sq: packed softmax (R <= 4), duplicated
# rows (5..8), two row blocks (9..32), four (33..64)
ROW_LAYOUTS = [(1, 1), (4, 1), (2, 2), (8, 1), (5, 1), (4, 3), (16, 1), (8, 4), (8, 5), (4, 16)]
FORMATS = ["int4", "bits3", "bits2", "asym32", "asym128"]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("G,Sq", ROW_LAYOUTS, ids=[f"G{g}xSq{s}" for g, s in ROW_LAYOUTS])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_few_keys_outlier_v(fmt, G, Sq, D):
    """A handful of keys (attention on 2..9 keys) over outlier-channel V."""
    if fmt == "asym128" and D == 64:
        pytest.skip("groups of 128 need D = 128")
    Hkv = 2
    errs = []
    for i, L in enumerate((2, 3, 5, 9)):
        q, cache, ref, _ = _decode_case(fmt, 100 * i + G * 7 + Sq + D, 1, G * Hkv, Hkv, Sq, L, D)
        scale = float(np.float32(1.0 / np.sqrt(D)))
        out, lse = _decode(fmt, q_to_dev(q), cache, L, scale)
        torch.cuda.synchronize()
        ro, rl = ref(q, L, scale)
        errs.append(compare(out, ro))
        assert compare(lse, rl)[0] < 1e-3
    mx = max(e[0] for e in errs)
    assert mx <= 4e-3 and max(e[1] for e in errs) <= 4e-4, f"{fmt} G={G} Sq={Sq} D={D}: max {mx:.3e}"


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("G,Sq", [(4, 1), (8, 1), (4, 3), (8, 5)], ids=["packed", "dup", "two_blocks", "four_blocks"])
@pytest.mark.parametrize("ns", [1, 3])
def test_decode_dominant_key_outlier_v(fmt, G, Sq, ns):
    """One key leads every score by ~6 (natural log units) among 300 keys whose
    outlier-channel V values reach ~100; splits 1 and 3 (the dominant key
    sits in one split)."""
    D, Hkv, L = 128, 2, 300
    q, cache, ref, _ = _decode_case(fmt, G * 10 + Sq + ns, 2, G * Hkv, Hkv, Sq, L, D, dominant=(217, 6.0))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse = _decode(fmt, q_to_dev(q), cache, L, scale, ns)
    torch.cuda.synchronize()
    ro, rl = ref(q, L, scale)
    assert_close(out, ro, f"{fmt} G={G} Sq={Sq} ns={ns}")
    assert compare(lse, rl)[0] < 1e-3


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_early_causal_rows_outlier_v(fmt, D):
    """Causal prefill: row i sees i + 1 keys, so the first rows attend a few
    outlier-channel V rows; every row is compared."""
    if fmt == "asym128" and D == 64:
        pytest.skip("groups of 128 need D = 128")
    B, Hq, Hkv, L = 1, 8, 2, 300
    q, cache, ref, _ = _decode_case(fmt, 31 + D, B, Hq, Hkv, L, L, D)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse = _prefill(fmt, q_to_dev(q), cache, L, True, scale)
    torch.cuda.synchronize()
    ro, rl = ref(q, L, scale, causal=True)
    assert_close(out, ro, f"{fmt} D={D}")
    assert compare(lse, rl)[0] < 1e-3


@pytest.mark.parametrize("fmt", ["int4", "bits3", "asym64"])
def test_prefill_dominant_key_outlier_v(fmt):
    """Non-causal prefill where one key dominates every row's scores."""
    B, Hq, Hkv, Sq, L, D = 1, 8, 2, 150, 400, 128
    q, cache, ref, _ = _decode_case(fmt, 77, B, Hq, Hkv, Sq, L, D, dominant=(333, 6.0))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse = _prefill(fmt, q_to_dev(q), cache, L, False, scale)
    torch.cuda.synchronize()
    ro, rl = ref(q, L, scale)
    assert_close(out, ro, fmt)



@pytest.mark.parametrize("fmt", ["int4", "bits3", "asym32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_outlier_rows_late_keys(fmt, causal, D):
    """Large V scales only among the last keys, which a dominant key makes the
    rows attend, in a cache of odd capacity (so the V scale rows of every
    head after the first start off a 16-byte boundary): each workgroup's scan
    of its keys' V scales must reach the last tile, and no further than its
    own keys."""
    rng = np.random.default_rng(90 + D + 2 * causal + len(fmt))
    B, Hq, Hkv, L, C = 2, 6, 3, 650, 701
    Sq = L if causal else 130
    q, k, v = _raw(rng, B, Hq, Hkv, Sq, C, D, vgain=1.0, dominant=(L - 3, 6.0))
    v[:, :, L - 6:L] *= np.float32(40.0)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    if fmt == "int4":
        kc, ks = oracle.quantize_rows(k)
        vc, vs = oracle.quantize_rows(v)
        ro, rl = oracle.attention(q, kc, ks, vc, vs, L, scale, causal=causal)
        cache = _sym_dev(kc, ks, vc, vs)
    elif fmt == "bits3":
        kc, ks = oracle.quantize_rows_bits(k, 3)
        vc, vs = oracle.quantize_rows_bits(v, 3)
        ro, rl = oracle.attention_bits(q, kc, ks, vc, vs, L, scale, 3, causal=causal)
        cache = _sym_dev(kc, ks, vc, vs)
    else:
        arrs = list(oracle.quantize_rows_asym(k, 32)) + list(oracle.quantize_rows_asym(v, 32))
        ro, rl = oracle.attention_asym(q, *arrs, L, scale, 32, causal=causal)
        cache = _asym_dev(arrs, 32)
    out, lse = _prefill(fmt, q_to_dev(q), cache, L, causal, scale)
    torch.cuda.synchronize()
    assert_close(out, ro, f"{fmt} causal={causal} D={D}")
    assert compare(lse, rl)[0] < 1e-3

def _chunked_outlier_rows(rng, B, Hkv, L, D, every):
    """V rows N(0, 1), except every `every`-th 32-token chunk holds rows x40: a
    wave meets chunks with and without large V scales in one split."""
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    for c0 in range(0, L, 32 * every):
        v[:, :, c0:c0 + 32] *= np.float32(40.0)
    return v


@pytest.mark.parametrize("G,Sq", [(4, 1), (1, 1), (8, 1), (4, 3)], ids=["packed", "packed_1row", "dup", "two_blocks"])
def test_decode_mixed_chunks(G, Sq):
    """Large V scales in some chunks only: the low-half columns must hold
    nothing from the other chunks."""
    rng = np.random.default_rng(G + Sq)
    B, Hkv, L, D = 2, 2, 2000, 128
    q = f32_to_bf16_bits(rng.standard_normal((B, G * Hkv, Sq, D)).astype(np.float32) * np.float32(2.0))
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    v = _chunked_outlier_rows(rng, B, Hkv, L, D, 5)
    kc, ks = oracle.quantize_rows(k)
    vc, vs = oracle.quantize_rows(v)
    for ns in (1, 4):
        out = qkv.decode(q_to_dev(q), _sym_dev(kc, ks, vc, vs), L, softmax_scale=0.2, num_splits=ns)
        torch.cuda.synchronize()
        ro, _ = oracle.attention(q, kc, ks, vc, vs, L, 0.2)
        assert_close(out, ro, f"G={G} Sq={Sq} ns={ns}")


@pytest.mark.parametrize("G,Sq", [(4, 1), (2, 1), (1, 3), (4, 2)], ids=["R4", "R2", "R3", "R8"])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_append_and_paged_outlier_v(G, Sq, D):
    """The fused append (new rows quantized in the kernel) and the paged cache
    over outlier-channel V with few keys, for 2, 3, 4 (packed softmax) and 8
    (duplicated rows) query rows per group."""
    rng = np.random.default_rng(5 + G + Sq + D)
    B, Hkv, P = 2, 2, 32
    Hq = G * Hkv
    for L in (3, 40):
        q, k, v = _raw(rng, B, Hq, Hkv, Sq, L, D)
        kc, ks = oracle.quantize_rows(k)
        vc, vs = oracle.quantize_rows(v)
        ro, _ = oracle.attention(q, kc, ks, vc, vs, L, 0.09)
        # fused append of the last row
        cache = _sym_dev(kc, ks, vc, vs)
        out = qkv.decode_append(q_to_dev(q), torch.from_numpy(k[:, :, -1:].copy()).to(DEV),
                                torch.from_numpy(v[:, :, -1:].copy()).to(DEV), cache, L - 1, softmax_scale=0.09)
        torch.cuda.synchronize()
        assert_close(out, ro, f"append L={L}")
        # paged: sequence b's pages in reverse order of a pool
        npg = -(-L // P)
        pool_k = np.zeros((B * npg, Hkv, P, D // 2), np.uint8)
        pool_ks = np.zeros((B * npg, Hkv, P), np.uint16)
        pool_v, pool_vs = pool_k.copy(), pool_ks.copy()
        table = np.zeros((B, npg), np.int32)
        for b in range(B):
            for i in range(npg):
                pid = B * npg - 1 - (b * npg + i)
                table[b, i] = pid
                n = min(P, L - i * P)
                pool_k[pid, :, :n], pool_ks[pid, :, :n] = kc[b, :, i * P:i * P + n], ks[b, :, i * P:i * P + n]
                pool_v[pid, :, :n], pool_vs[pid, :, :n] = vc[b, :, i * P:i * P + n], vs[b, :, i * P:i * P + n]
        lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
        out = qkv.decode_paged(q_to_dev(q), _sym_dev(pool_k, pool_ks, pool_v, pool_vs), lens,
                               torch.from_numpy(table).to(DEV), max_kv_len=L, softmax_scale=0.09)
        torch.cuda.synchronize()
        assert_close(out, ro, f"paged L={L}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_large_v_magnitudes(causal, D):
    """V row absmax up to ~4.5e5 (fp16 scales up to ~64000) and scores that move
    by more than 2^8 between tiles: outputs stay finite and within 1e-5 of the
    oracle relative to the largest |v|."""
    rng = np.random.default_rng(D + causal)
    B, Hq, Hkv, L = 1, 4, 2, 500
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, L, D)).astype(np.float32))
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32) * np.linspace(1, 6, L, dtype=np.float32)[None, None, :, None]
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    v /= np.abs(v).max(axis=-1, keepdims=True)
    v *= np.float32(7 * 64000) * rng.uniform(0.05, 1.0, size=(B, Hkv, L, 1)).astype(np.float32)
    kc, ks = oracle.quantize_rows(k)
    vc, vs = oracle.quantize_rows(v)
    assert vs.view(np.float16).max() > 60000
    scale = float(np.float32(1.0 / np.sqrt(D)))
    ro, _ = oracle.attention(q, kc, ks, vc, vs, L, scale, causal=causal)
    vmax = float(np.abs(oracle.dequantize_rows(vc, vs)).max())
    out = qkv.prefill(q_to_dev(q), _sym_dev(kc, ks, vc, vs), L, causal, softmax_scale=scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "prefill output not finite"
    rel = compare(out, ro)[0] / vmax
    assert rel <= 1e-5, f"prefill relative error {rel:.2e}"
    if not causal:
        out = qkv.decode(q_to_dev(q[:, :, :3]), _sym_dev(kc, ks, vc, vs), L, softmax_scale=scale)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all()), "decode output not finite"
        rel = compare(out, ro[:, :, :3])[0] / vmax
        assert rel <= 1e-5, f"decode relative error {rel:.2e}"


@pytest.mark.parametrize("qmax_log2", [16, 22, 60])
def test_query_past_fp16_range(qmax_log2):
    """Query elements up to 2^qmax_log2 (beyond fp16's 65504), softmax scale
    2^-qmax_log2 / sqrt(D): the kernels shift the query by an exact power of
    two into fp16 range, so scores and outputs match the oracle.  One row per
    group keeps ordinary magnitudes."""
    rng = np.random.default_rng(qmax_log2)
    B, Hq, Hkv, D, L = 2, 8, 2, 128, 700
    qf = rng.standard_normal((B, Hq, 5, D)).astype(np.float32) * np.float32(2.0 ** (qmax_log2 - 2))
    qf[:, 0] = rng.standard_normal((B, 5, D)).astype(np.float32)
    q = f32_to_bf16_bits(qf)
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    kc, ks = oracle.quantize_rows(k)
    vc, vs = oracle.quantize_rows(v)
    scale = float(np.float32(2.0 ** -qmax_log2 / np.sqrt(D)))
    cache = _sym_dev(kc, ks, vc, vs)
    for Sq in (1, 5):
        qs = np.ascontiguousarray(q[:, :, :Sq])
        out, lse = qkv.decode(q_to_dev(qs), cache, L, softmax_scale=scale, return_lse=True)
        torch.cuda.synchronize()
        ro, rl = oracle.attention(qs, kc, ks, vc, vs, L, scale)
        assert_close(out, ro, f"decode Sq={Sq}")
        assert compare(lse, rl)[0] < 1e-3
    out, lse = qkv.prefill(q_to_dev(q), cache, L, True, softmax_scale=scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, kc, ks, vc, vs, L, scale, causal=True)
    assert_close(out, ro, "prefill")
    assert compare(lse, rl)[0] < 1e-3

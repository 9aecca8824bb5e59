"""GPU parity of the short-sequence prefill (kv_len <= 256, D = 64, int4 rows:
one workgroup per head, whole key range in LDS) against the fp64 oracle:
ragged key counts around every padding boundary (8-token V rows, complete
and partial 16-token PV groups, 32-token key blocks), query counts from 1 to
256 (one or two 32-row blocks per wave), causal with Sq <= kv_len, GQA and head maps, channel-outlier V under
concentrated attention (hi/lo P~), V scales near the fp16 limit, and
queries past fp16 range."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_flashattention_amd as qkv
from gpu_helpers import DEV, assert_close, cache_to_dev, compare, q_to_dev, random_case
from qkv_inputs import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, Sq, L, C, causal
    (1, 2, 2, 1, 1, 1, True),
    (1, 2, 1, 1, 1, 9, False),
    (1, 4, 2, 7, 8, 8, False),
    (1, 4, 4, 31, 31, 33, True),
    (1, 4, 4, 32, 32, 32, True),
    (1, 4, 4, 33, 33, 40, False),
    (1, 2, 2, 5, 16, 16, True),
    (1, 2, 2, 17, 240, 240, False),    # 240 % 16 == 0: V stride 248
    (1, 8, 2, 40, 248, 249, False),
    (1, 3, 1, 100, 255, 301, False),
    (1, 2, 2, 256, 256, 256, True),
    (1, 2, 2, 256, 256, 256, False),
    (1, 2, 2, 250, 256, 300, True),    # Sq < kv_len: bottom-right causal
    (2, 4, 4, 197, 197, 197, False),   # ViT-B row count
    (2, 6, 3, 129, 129, 140, True),
    (3, 12, 12, 197, 197, 197, False),
]


@pytest.mark.parametrize("outliers", [False, True], ids=["normal", "outlier_channels"])
@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_short_prefill_matches_oracle(case, outliers):
    B, Hq, Hkv, Sq, L, C, causal = case
    D = 64
    q, kc, ks, vc, vs = random_case(sum(case) + 7 * outliers, B, Hq, Hkv, Sq, L, D, C, outliers=outliers)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse = qkv.prefill(q_to_dev(q), cache_to_dev(kc, ks, vc, vs), L, causal, softmax_scale=scale,
                           return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, kc, ks, vc, vs, L, scale, causal)
    assert_close(out, ro, str(case))
    assert compare(lse, rl)[0] < 1e-3


def _outlier_case(rng, B, Hq, Hkv, Sq, L, dominant, vgain=1.0, late=False):
    """x8 outlier channels in K and V; V rows x40 at the dominant key (or the
    last 6 keys) so that P~ needs its hi/lo form; the dominant key leads every
    row's scores by about 6 (natural log units)."""
    D = 64
    q = rng.standard_normal((B, Hq, Sq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    v = (rng.standard_normal((B, Hkv, L, D)) * vgain).astype(np.float32)
    for t in (k, v):
        t[..., rng.choice(D, size=2, replace=False)] *= np.float32(8.0)
    G = Hq // Hkv
    for g in range(Hkv):
        qd = q[:, g * G:(g + 1) * G].mean(axis=(1, 2))
        nrm = np.linalg.norm(qd, axis=-1, keepdims=True)
        k[:, g, dominant] = qd / nrm * np.float32(6.0 * np.sqrt(D) / max(float(nrm.min()), 1e-3))
    if late:
        v[:, :, L - 6:L] *= np.float32(40.0)
    else:
        v[:, :, dominant] *= np.float32(40.0)
    return f32_to_bf16_bits(q), k, v


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("L,dominant,late", [(197, 150, False), (64, 3, False), (250, 246, True), (9, 8, True)])
def test_short_prefill_outlier_v_concentrated(causal, L, dominant, late):
    """Channel-outlier V rows that every row attends almost alone: one fp16
    rounding of P~ would miss the tolerance, so these pass only with P~ as an
    fp16 hi/lo pair."""
    rng = np.random.default_rng(L + dominant + causal)
    B, Hq, Hkv, Sq = 2, 6, 2, L
    q, k, v = _outlier_case(rng, B, Hq, Hkv, Sq, L, dominant, late=late)
    kc, ks = oracle.quantize_rows(k)
    vc, vs = oracle.quantize_rows(v)
    scale = 0.125
    out, lse = qkv.prefill(q_to_dev(q), cache_to_dev(kc, ks, vc, vs), L, causal, softmax_scale=scale,
                           return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, kc, ks, vc, vs, L, scale, causal)
    assert_close(out, ro, f"L={L} causal={causal}")
    assert compare(lse, rl)[0] < 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_short_prefill_large_v_magnitudes(causal):
    """V row absmax up to ~4.5e5 (fp16 scales near 64000) and key scales that
    grow along the keys: outputs finite and within 1e-5 of the oracle relative
    to the largest |v|."""
    rng = np.random.default_rng(11 + causal)
    B, Hq, Hkv, L, D = 1, 4, 2, 230, 64
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, L, D)).astype(np.float32))
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32) * np.linspace(1, 6, L, dtype=np.float32)[None, None, :, None]
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    v /= np.abs(v).max(axis=-1, keepdims=True)
    v *= np.float32(7 * 64000) * rng.uniform(0.05, 1.0, size=(B, Hkv, L, 1)).astype(np.float32)
    kc, ks = oracle.quantize_rows(k)
    vc, vs = oracle.quantize_rows(v)
    assert vs.view(np.float16).max() > 60000
    scale = 0.125
    ro, _ = oracle.attention(q, kc, ks, vc, vs, L, scale, causal=causal)
    vmax = float(np.abs(oracle.dequantize_rows(vc, vs)).max())
    out = qkv.prefill(q_to_dev(q), cache_to_dev(kc, ks, vc, vs), L, causal, softmax_scale=scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    assert compare(out, ro)[0] / vmax <= 1e-5


@pytest.mark.parametrize("qmax_log2", [16, 40])
def test_short_prefill_query_past_fp16_range(qmax_log2):
    rng = np.random.default_rng(qmax_log2)
    B, Hq, Hkv, Sq, L, D = 2, 4, 2, 150, 150, 64
    qf = rng.standard_normal((B, Hq, Sq, D)).astype(np.float32) * np.float32(2.0 ** (qmax_log2 - 2))
    qf[:, 0] = rng.standard_normal((B, Sq, D)).astype(np.float32)
    q = f32_to_bf16_bits(qf)
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    kc, ks = oracle.quantize_rows(k)
    vc, vs = oracle.quantize_rows(v)
    scale = float(np.float32(2.0 ** -qmax_log2 / np.sqrt(D)))
    out, lse = qkv.prefill(q_to_dev(q), cache_to_dev(kc, ks, vc, vs), L, True, softmax_scale=scale,
                           return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, kc, ks, vc, vs, L, scale, causal=True)
    assert_close(out, ro, f"qmax 2^{qmax_log2}")
    assert compare(lse, rl)[0] < 1e-3


def test_short_prefill_head_map_matches_plain():
    """A head map over a cache holding two of a layer's four KV heads writes
    exactly those heads' query rows, equal to the plain call on that cache."""
    rng_seed = 5
    B, Hkv_all, G, Sq, L, D = 2, 4, 3, 120, 180, 64
    q, kc, ks, vc, vs = random_case(rng_seed, B, Hkv_all * G, Hkv_all, Sq, L, D)
    heads = np.array([3, 1], dtype=np.int32)
    sub = tuple(np.ascontiguousarray(a[:, heads]) for a in (kc, ks, vc, vs))
    cache = cache_to_dev(*sub)
    out = torch.full((B, Hkv_all * G, Sq, D), float("nan"), device=DEV)
    qkv.prefill_heads(q_to_dev(q), cache, torch.from_numpy(heads).to(DEV), Hkv_all, L, False, out,
                      softmax_scale=0.125)
    qsub = np.ascontiguousarray(np.concatenate([q[:, h * G:(h + 1) * G] for h in heads], axis=1))
    ref = qkv.prefill(q_to_dev(qsub), cache, L, False, softmax_scale=0.125)
    torch.cuda.synchronize()
    for i, h in enumerate(heads):
        assert torch.equal(out[:, h * G:(h + 1) * G], ref[:, i * G:(i + 1) * G])
    others = [h for h in range(Hkv_all) if h not in heads]
    for h in others:
        assert bool(torch.isnan(out[:, h * G:(h + 1) * G]).all())

"""GPU prefill parity (causal and not) against the fp64 oracle (max-abs 4e-3, mean-abs 4e-4)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_flashattention_amd as qkv
from gpu_helpers import (DEV, assert_close, cache_to_dev, compare, full_workload, oracle_cache, q_to_dev,
                         random_case)
from qkv_inputs import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _run(q, cache, L, causal, scale):
    out, lse = qkv.prefill(q_to_dev(q), cache_to_dev(*cache), L, causal, softmax_scale=scale, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    # B, Hq, Hkv, Sq, L, C, D, causal
    (1, 2, 2, 1, 1, 1, 64, True),
    (2, 4, 4, 197, 197, 197, 64, False),
    (1, 8, 2, 1000, 1000, 1000, 128, True),
    (1, 8, 2, 1000, 1000, 1024, 128, False),
    (1, 4, 1, 300, 1000, 1000, 128, True),     # Sq < kv_len: bottom-right causal
    (2, 6, 3, 129, 129, 140, 64, True),
    (1, 16, 2, 64, 64, 64, 128, True),
    (1, 4, 4, 5, 700, 700, 64, False),
    (1, 8, 8, 255, 513, 513, 64, True),
]


@pytest.mark.parametrize("outliers", [False, True], ids=["normal", "outlier_channels"])
@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_prefill_matches_oracle(case, outliers):
    B, Hq, Hkv, Sq, L, C, D, causal = case
    q, kc, ks, vc, vs = random_case(sum(case[:7]), B, Hq, Hkv, Sq, L, D, C, outliers=outliers)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse = _run(q, (kc, ks, vc, vs), L, causal, scale)
    ro, rl = oracle.attention(q, kc, ks, vc, vs, L, scale, causal)
    assert_close(out, ro, str(case))
    assert compare(lse, rl)[0] < 1e-3


def test_prefill_deterministic_and_no_nan():
    q, kc, ks, vc, vs = random_case(3, 1, 8, 2, 700, 700, 128)
    a, la = _run(q, (kc, ks, vc, vs), 700, True, 0.09)
    b, lb = _run(q, (kc, ks, vc, vs), 700, True, 0.09)
    assert torch.equal(a, b) and torch.equal(la, lb)
    out = torch.full((1, 8, 700, 128), float("nan"), device=DEV)
    qkv.prefill(q_to_dev(q), cache_to_dev(kc, ks, vc, vs), 700, True, softmax_scale=0.09, out=out)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(out).any())


def test_full_size_vit():
    w, q, kc, ks, vc, vs = full_workload(1)
    out, lse = _run(q, (kc, ks, vc, vs), w.L, w.causal, w.softmax_scale)
    ro, rl = oracle.attention(q, kc, ks, vc, vs, w.L, w.softmax_scale, w.causal)
    mx, mn = assert_close(out, ro, w.name)
    print(f"{w.name}: max {mx:.3e} mean {mn:.3e}")


def test_full_size_causal_prefill_sampled():
    """16K causal GQA prefill at full size; the oracle computes sampled rows of every head."""
    w, q, kc, ks, vc, vs = full_workload(4)
    out, lse = _run(q, (kc, ks, vc, vs), w.L, True, w.softmax_scale)
    assert not bool(torch.isnan(out).any())
    rng = np.random.default_rng(0)
    rows = sorted(set([0, 1, 2, 63, 64, 127, 128, 129, 1000, 4095, 4096, 8191, 12345, 16382, 16383]
                      + list(rng.integers(0, w.Sq, 17))))
    heads = [(0, h) for h in range(w.Hq)]
    ro, rl = oracle.attention(q, kc, ks, vc, vs, w.L, w.softmax_scale, True, heads=heads, rows=rows)
    mx, mn = assert_close(out, ro, w.name)
    print(f"{w.name}: sampled max {mx:.3e} mean {mn:.3e}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("trend", ["rising", "falling"])
def test_prefill_score_trends(D, causal, trend):
    """K rows scaled by a factor that grows (or shrinks) 40x along the keys,
    so a row's running maximum keeps moving by far more than 2^8 between
    tiles: every rescale decision of the online softmax is exercised (a missed
    one overflows fp16 probabilities into inf/NaN)."""
    rng = np.random.default_rng(D + 2 * causal + (trend == "rising"))
    B, Hq, Hkv, Sq, L = 1, 4, 2, 700, 900
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, Sq, D)).astype(np.float32))
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    f = np.linspace(1.0, 40.0, L, dtype=np.float32)
    k *= (f if trend == "rising" else f[::-1])[None, None, :, None]
    kc, ks, vc, vs = oracle_cache(k, v, L + 3, seed=D)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse = _run(q, (kc, ks, vc, vs), L, causal, scale)
    assert not bool(torch.isnan(out).any()) and not bool(torch.isinf(out).any())
    ro, rl = oracle.attention(q, kc, ks, vc, vs, L, scale, causal)
    assert_close(out, ro, f"{trend} D={D} causal={causal}")
    assert compare(lse, rl)[0] < 1e-3

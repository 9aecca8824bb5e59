"""GPU split-K decode parity against the fp64 oracle (max-abs 4e-3, mean-abs 4e-4).

The GPU consumes oracle-quantized caches (uploaded), so attention parity does
not depend on the GPU quantizer.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_flashattention_amd as qkv
from gpu_helpers import (DEV, MAX_ABS_TOL, MEAN_ABS_TOL, assert_close, cache_to_dev, compare,
                         full_workload, q_to_dev, random_case)

pytestmark = pytest.mark.gpu


def _run(q, cache, L, scale, ns=0, lse=True):
    out, l = qkv.decode(q_to_dev(q), cache_to_dev(*cache), L, softmax_scale=scale, num_splits=ns,
                        return_lse=True)
    torch.cuda.synchronize()
    return out, l


CASES = [
    # B, Hq, Hkv, Sq, L, C, D
    (1, 2, 2, 1, 256, 256, 64),
    (2, 8, 2, 1, 1000, 1024, 128),
    (1, 8, 8, 1, 33, 40, 64),
    (2, 32, 8, 2, 777, 800, 128),
    (1, 64, 8, 1, 4097, 4100, 128),
    (1, 8, 2, 5, 129, 129, 64),      # 20 rows per group -> two 16-row blocks
    (1, 4, 1, 16, 300, 300, 128),    # 64 rows per group -> four blocks
    (3, 12, 4, 3, 2049, 2100, 128),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
@pytest.mark.parametrize("ns", [0, 1, 3])
def test_decode_matches_oracle(case, ns):
    B, Hq, Hkv, Sq, L, C, D = case
    q, kc, ks, vc, vs = random_case(sum(case), B, Hq, Hkv, Sq, L, D, C)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse = _run(q, (kc, ks, vc, vs), L, scale, ns)
    ro, rl = oracle.attention(q, kc, ks, vc, vs, L, scale)
    assert_close(out, ro, f"out {case} ns={ns}")
    mx, _ = compare(lse, rl)
    assert mx < 1e-3, mx


@pytest.mark.parametrize("L", [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 197])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_kv_len_edges(L, D):
    q, kc, ks, vc, vs = random_case(L + D, 2, 4, 2, 1, L, D, C=L + 5)
    out, lse = _run(q, (kc, ks, vc, vs), L, 0.125)
    ro, rl = oracle.attention(q, kc, ks, vc, vs, L, 0.125)
    assert_close(out, ro, f"L={L} D={D}")


def test_split_counts_agree_and_are_deterministic():
    q, kc, ks, vc, vs = random_case(5, 2, 16, 4, 1, 3000, 128, C=3000, outliers=True)
    ro, _ = oracle.attention(q, kc, ks, vc, vs, 3000, 0.088)
    outs = {}
    for ns in (1, 2, 7, 0, 94):
        a, _ = _run(q, (kc, ks, vc, vs), 3000, 0.088, ns)
        b, _ = _run(q, (kc, ks, vc, vs), 3000, 0.088, ns)
        assert torch.equal(a, b), f"run-to-run difference at ns={ns}"
        assert_close(a, ro, f"ns={ns}")
        outs[ns] = a
    for ns, a in outs.items():
        assert float((a - outs[1]).abs().max()) < MAX_ABS_TOL


def test_gqa_equals_repeated_kv():
    q, kc, ks, vc, vs = random_case(6, 1, 16, 2, 2, 500, 128)
    a, _ = _run(q, (kc, ks, vc, vs), 500, 0.1)
    rep = lambda x: np.repeat(x, 8, axis=1)
    b, _ = _run(q, (rep(kc), rep(ks), rep(vc), rep(vs)), 500, 0.1)
    assert float((a - b).abs().max()) < 1e-5


def test_output_buffers_prefilled_with_nan():
    q, kc, ks, vc, vs = random_case(7, 2, 8, 2, 1, 900, 128)
    out = torch.full((2, 8, 1, 128), float("nan"), device=DEV)
    lse = torch.full((2, 8, 1), float("nan"), device=DEV)
    qkv.decode(q_to_dev(q), cache_to_dev(kc, ks, vc, vs), 900, softmax_scale=0.1, out=out, lse=lse,
               return_lse=True)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(out).any()) and not bool(torch.isnan(lse).any())


@pytest.mark.parametrize("index", [0, 2, 3])
def test_full_size_decode_workloads(index):
    """tiny decode, Llama-3-8B decode (outliers) and 128K decode, at full size,
    auto split count (the benchmark's launch configuration), every head."""
    w, q, kc, ks, vc, vs = full_workload(index)
    out, lse = _run(q, (kc, ks, vc, vs), w.L, w.softmax_scale)
    ro, rl = oracle.attention(q, kc, ks, vc, vs, w.L, w.softmax_scale)
    mx, mn = assert_close(out, ro, w.name)
    print(f"{w.name}: max {mx:.3e} mean {mn:.3e}")
    assert compare(lse, rl)[0] < 1e-3

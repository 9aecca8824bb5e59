"""The seeded input generator: determinism, shapes, bf16 rounding, outlier structure."""
import numpy as np
import torch

from qkv_inputs import (WORKLOADS, f32_to_bf16_bits, bf16_bits_to_f32, make_qkv, pool_rows, ragged_layout,
                        workload)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-38).astype(np.float32),
                        np.array([0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workload_table():
    assert [w.name for w in WORKLOADS] == ["tiny_decode", "vit_b_selfattn", "llama3_8b_decode",
                                           "long_context_decode", "causal_prefill_16k", "ragged_paged_decode"]
    for w in WORKLOADS:
        assert w.Hq % w.Hkv == 0 and w.D in (64, 128)
    assert workload(2).G == 4 and workload(3).G == 8


def test_deterministic_and_shaped():
    w = workload(0)
    q1, k1, v1 = make_qkv(w, seed=3)
    q2, k2, v2 = make_qkv(w, seed=3)
    assert np.array_equal(q1, q2) and np.array_equal(k1, k2) and np.array_equal(v1, v2)
    assert q1.shape == (1, 2, 1, 64) and q1.dtype == np.uint16
    assert k1.shape == (1, 2, 256, 64) and k1.dtype == np.float32
    q3, _, _ = make_qkv(w, seed=4)
    assert not np.array_equal(q1, q3)


def test_outlier_channels():
    w = workload(2).scaled(B=2, L=64)
    _, k, v = make_qkv(w, seed=0)
    for t in (k, v):
        rms = np.sqrt((t.astype(np.float64) ** 2).mean(axis=(0, 2)))   # [Hkv, D]
        big = rms > 4.0
        assert big.sum() == 10                   # 1% of 8*128 channels, x8


def test_ragged_layout():
    w = workload("ragged_paged_decode")
    lens, table, num_pages = ragged_layout(w, seed=1)
    assert lens.dtype == np.int32 and lens.shape == (w.B,)
    assert lens.min() >= w.len_min and lens.max() <= w.L
    l2, t2, n2 = ragged_layout(w, seed=1)
    assert np.array_equal(lens, l2) and np.array_equal(table, t2) and n2 == num_pages
    P = w.page_size
    used = [table[b, :-(-int(L) // P)] for b, L in enumerate(lens)]
    ids = np.concatenate(used)
    assert sorted(ids.tolist()) == list(range(num_pages))    # every page exactly once
    for b, L in enumerate(lens):
        assert np.all(table[b, -(-int(L) // P):] == -1)
    small = w.scaled(B=3, L=100, len_min=10, page_size=32)
    it = list(pool_rows(small, 5, 2, seed=0))
    assert [p0 for p0, _, _ in it] == [0, 2, 4]
    assert it[0][1].shape == (2, small.Hkv, 32, small.D) and it[2][1].shape == (1, small.Hkv, 32, small.D)

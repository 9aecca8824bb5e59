"""GPU quantize-and-append parity: byte-exact codes and scales against the oracle.

Rows outside [pos, pos+T) of the cache are pre-filled with a canary and must
stay untouched.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import quantized_kv_flashattention_amd as qkv
from gpu_helpers import DEV, full_workload
from qkv_inputs import workload, make_qkv

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantizer_rows.txt")


def _golden():
    cases, cur = [], {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split(":", 1)
        if k == "row":
            cur = {"row": np.array([float(t) for t in v.split()], np.float32)}
        elif k == "scale":
            cur["scale"] = int(v, 16)
        else:
            cur["bytes"] = bytes(int(t, 16) for t in v.split())
            cases.append(cur)
    return cases


def _gpu_quantize(src: np.ndarray, C: int, pos: int):
    B, H, T, D = src.shape
    codes = torch.full((B, H, C, D // 2), 0xA5, dtype=torch.uint8, device=DEV)
    scales = torch.full((B, H, C), 0, dtype=torch.int16, device=DEV)
    scales.fill_(-23131)  # 0xA5A5
    scales = scales.view(torch.float16)
    qkv.quantize_append(torch.from_numpy(src).to(DEV), codes, scales, pos)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.view(torch.int16).cpu().numpy().view(np.uint16)


def _check(src, C, pos):
    T = src.shape[2]
    codes, scales = _gpu_quantize(src, C, pos)
    rc, rs = oracle.quantize_rows(src)
    assert np.array_equal(codes[:, :, pos:pos + T], rc)
    assert np.array_equal(scales[:, :, pos:pos + T], rs)
    assert np.all(codes[:, :, :pos] == 0xA5) and np.all(codes[:, :, pos + T:] == 0xA5)
    assert np.all(scales[:, :, :pos] == 0xA5A5) and np.all(scales[:, :, pos + T:] == 0xA5A5)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("offset", [0, 40])
def test_golden_rows(D, offset):
    cases = _golden()
    rows = np.zeros((1, 1, len(cases), D), np.float32)
    for i, c in enumerate(cases):
        rows[0, 0, i, offset:offset + 8] = c["row"]
    codes, scales = _gpu_quantize(rows, len(cases), 0)
    for i, c in enumerate(cases):
        assert int(scales[0, 0, i]) == c["scale"], i
        got = codes[0, 0, i].tobytes()
        assert got[offset // 2: offset // 2 + 4] == c["bytes"], i
        assert got[:offset // 2] == bytes(offset // 2) and got[offset // 2 + 4:] == bytes(D // 2 - offset // 2 - 4)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T,C,pos", [(1, 5, 4), (37, 50, 13), (256, 256, 0), (1000, 1100, 17)])
def test_random_rows(D, T, C, pos):
    rng = np.random.default_rng(T + D)
    src = rng.standard_normal((2, 3, T, D)).astype(np.float32)
    # mix in wide magnitudes, exact zeros, subnormal-scale rows and exact ties
    src[0, 0] *= np.float32(2.0) ** rng.integers(-30, 12, size=(T, 1)).astype(np.float32)
    src[0, 1, ::3] = 0
    src[1, 0] *= np.float32(1e-6)
    ties = (rng.integers(-7, 7, size=(T, D)) + 0.5).astype(np.float32)
    ties[:, 0] = 7.0
    src[1, 1] = ties * np.float32(0.375)
    _check(src, C, pos)


def test_zero_rows_noop():
    codes = torch.full((1, 1, 4, 32), 0xA5, dtype=torch.uint8, device=DEV)
    scales = torch.zeros((1, 1, 4), dtype=torch.float16, device=DEV)
    qkv.quantize_append(torch.empty((1, 1, 0, 64), device=DEV), codes, scales, 4)
    torch.cuda.synchronize()
    assert bool((codes == 0xA5).all())


@pytest.mark.parametrize("index", [0, 1, 2, 3, 4])
def test_full_size_workloads(index):
    """K and V of every workload, at full size, quantized as one append each."""
    w, q, kc, ks, vc, vs = full_workload(index)
    _, k, v = make_qkv(w)
    for src, rc, rs in ((k, kc, ks), (v, vc, vs)):
        B, H, L, D = src.shape
        codes = torch.empty((B, H, L, D // 2), dtype=torch.uint8, device=DEV)
        scales = torch.empty((B, H, L), dtype=torch.float16, device=DEV)
        qkv.quantize_append(torch.from_numpy(src).to(DEV), codes, scales, 0)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), rc)
        assert np.array_equal(scales.view(torch.int16).cpu().numpy().view(np.uint16), rs)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T,C,pos", [(1, 9, 8), (300, 310, 5)])
def test_append_kv_matches_two_appends(D, T, C, pos):
    rng = np.random.default_rng(T * D)
    k = rng.standard_normal((3, 2, T, D)).astype(np.float32)
    v = (rng.standard_normal((3, 2, T, D)) * 3).astype(np.float32)
    cache = qkv.KVCache(*(torch.full(s, f, dtype=dt, device=DEV) for s, f, dt in (
        ((3, 2, C, D // 2), 0xA5, torch.uint8), ((3, 2, C), 1.5, torch.float16),
        ((3, 2, C, D // 2), 0x5A, torch.uint8), ((3, 2, C), -2.5, torch.float16))))
    qkv.quantize_append_kv(torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV), cache, pos)
    torch.cuda.synchronize()
    for src, codes, scales, fill_c, fill_s in ((k, cache.k_codes, cache.k_scales, 0xA5, 1.5),
                                               (v, cache.v_codes, cache.v_scales, 0x5A, -2.5)):
        rc, rs = oracle.quantize_rows(src)
        c = codes.cpu().numpy()
        s = scales.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(c[:, :, pos:pos + T], rc) and np.array_equal(s[:, :, pos:pos + T], rs)
        assert np.all(c[:, :, :pos] == fill_c) and np.all(c[:, :, pos + T:] == fill_c)
        fs = np.float16(fill_s).view(np.uint16)
        assert np.all(s[:, :, :pos] == fs) and np.all(s[:, :, pos + T:] == fs)

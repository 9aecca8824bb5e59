"""Shared helpers of the GPU parity tests: seeded inputs, oracle caches, upload, tolerances."""
from __future__ import annotations

import functools

import numpy as np
import torch

import oracle
import quantized_kv_flashattention_amd as qkv
from qkv_inputs import f32_to_bf16_bits, make_qkv, workload

MAX_ABS_TOL = 4e-3    # attention tolerance (max |gpu - oracle|)
MEAN_ABS_TOL = 4e-4   # attention tolerance (mean |gpu - oracle| over all compared elements)

DEV = "cuda"


def q_to_dev(q_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def cache_to_dev(kc, ks, vc, vs) -> qkv.KVCache:
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    h = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).to(DEV)
    return qkv.KVCache(t(kc), h(ks), t(vc), h(vs))


def oracle_cache(k: np.ndarray, v: np.ndarray, C: int | None = None, seed: int = 99):
    """Oracle-quantized cache of capacity C >= L; rows >= L hold random garbage."""
    B, H, L, D = k.shape
    C = C or L
    rng = np.random.default_rng(seed)
    out = []
    for t in (k, v):
        codes = rng.integers(0, 256, size=(B, H, C, D // 2), dtype=np.uint8)
        scales = rng.integers(0, 0x7800, size=(B, H, C), dtype=np.uint16)   # finite fp16 garbage
        qc, qs = oracle.quantize_rows(t)
        codes[:, :, :L] = qc
        scales[:, :, :L] = qs
        out += [codes, scales]
    return tuple(out)


def random_case(seed, B, Hq, Hkv, Sq, L, D, C=None, outliers=False):
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, Sq, D)).astype(np.float32))
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    if outliers:
        for t in (k, v):
            ch = rng.choice(Hkv * D, size=max(1, Hkv * D // 100), replace=False)
            for c in ch:
                t[:, c // D, :, c % D] *= np.float32(8)
    return (q,) + oracle_cache(k, v, C, seed + 1)


@functools.lru_cache(maxsize=1)
def full_workload(index: int, seed: int = 0):
    """(workload, q_bits, k_codes, k_scales, v_codes, v_scales) of a full-size workload."""
    w = workload(index)
    q, k, v = make_qkv(w, seed)
    kc, ks = oracle.quantize_rows(k)
    del k
    vc, vs = oracle.quantize_rows(v)
    del v
    return w, q, kc, ks, vc, vs


def compare(gpu: torch.Tensor, ref: np.ndarray, mask=None):
    """Return (max_abs, mean_abs) of gpu vs ref over entries where ref is not NaN."""
    g = gpu.detach().cpu().double().numpy()
    ok = ~np.isnan(ref) if mask is None else mask
    assert not np.any(np.isnan(g[ok])), "GPU output holds NaN"
    d = np.abs(g[ok] - ref[ok])
    return float(d.max()), float(d.mean())


def assert_close(gpu, ref, what=""):
    mx, mn = compare(gpu, ref)
    assert mx <= MAX_ABS_TOL and mn <= MEAN_ABS_TOL, f"{what}: max {mx:.3e} mean {mn:.3e}"
    return mx, mn

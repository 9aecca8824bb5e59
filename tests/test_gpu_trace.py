"""The measurement build (libqkvfa_trace.so: the same kernels plus decode
phase timestamps) computes what libqkvfa.so computes, and its timestamps
are ordered the way the decode kernel's phases run."""
import ctypes
import os

import numpy as np
import pytest
import torch

import quantized_kv_flashattention_amd as qkv
from gpu_helpers import cache_to_dev, q_to_dev, random_case

pytestmark = pytest.mark.gpu

TRACE_LIB = os.path.join(os.path.dirname(qkv.library_path()), "libqkvfa_trace.so")


@pytest.mark.skipif(not os.path.exists(TRACE_LIB), reason="libqkvfa_trace.so not built")
def test_trace_build_matches_and_orders_phases():
    B, Hq, Hkv, Sq, L, D = 2, 8, 2, 1, 3000, 128
    q, kc, ks, vc, vs = random_case(77, B, Hq, Hkv, Sq, L, D, C=L + 8)
    k_new = torch.randn(B, Hkv, 1, D, device="cuda")
    v_new = torch.randn(B, Hkv, 1, D, device="cuda")
    ns = 3
    outs = []
    plain = qkv._lib
    tl = ctypes.CDLL(TRACE_LIB)
    tl.qkv_trace_read.restype = ctypes.c_int
    tl.qkv_trace_read.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    try:
        for lib_path in (qkv.library_path(), TRACE_LIB):
            saved = qkv._LIB_PATH
            qkv._LIB_PATH = lib_path
            qkv._lib = qkv._load()
            qkv._LIB_PATH = saved
            cache = cache_to_dev(kc, ks, vc, vs)
            o, l = qkv.decode_append(q_to_dev(q), k_new, v_new, cache, L, softmax_scale=0.088, num_splits=ns,
                                     return_lse=True)
            torch.cuda.synchronize()
            outs.append((o, l, [t.clone() for t in cache.tensors()]))
    finally:
        qkv._lib = plain
    (o1, l1, c1), (o2, l2, c2) = outs
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "the trace build computes different outputs"
    for a, b in zip(c1, c2):
        assert torch.equal(a, b)
    n_wg = ns * B * Hkv
    buf = np.zeros((n_wg, 16), dtype=np.uint64)
    assert tl.qkv_trace_read(buf.ctypes.data, n_wg) == 0
    t = buf.astype(np.int64)
    # entry <= loop start <= every wave's end <= merge written <= ticket <= exit
    assert np.all(t[:, 0] <= t[:, 1])
    assert np.all(t[:, 1][:, None] <= t[:, 2:10])
    assert np.all(t[:, 2:10].max(axis=1) <= t[:, 10])
    assert np.all(t[:, 10] <= t[:, 11]) and np.all(t[:, 11] <= t[:, 12])
    # exactly one workgroup of each (batch, KV head) merged its splits
    merged = buf[:, 13].reshape(ns, B * Hkv)
    assert np.all(merged.sum(axis=0) == 1)
    # one launch spans microseconds, not more than a second (100 MHz clock)
    assert 0 < t[:, 12].max() - t[:, 0].min() < 100_000_000

"""qkv_decode_noalloc (split partials in the library's static per-device
scratch) against qkv_decode (caller's workspace): same kernels and split
plan, so the outputs and log-sum-exps must agree bit for bit, also on a
second, smaller call right after the first (the scratch keeps the previous
call's contents) and on a repeat of the first shape (the tickets were left
at zero)."""
import pytest
import torch

import oracle
import quantized_kv_flashattention_amd as qkv
from gpu_helpers import DEV, assert_close, cache_to_dev, q_to_dev, random_case

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, Sq, L, D, num_splits): the larger shape first
SHAPES = [(4, 32, 8, 1, 3000, 128, 0), (2, 8, 2, 2, 700, 64, 3)]


def _run(shape, seed):
    B, Hq, Hkv, Sq, L, D, ns = shape
    q, kc, ks, vc, vs = random_case(seed, B, Hq, Hkv, Sq, L, D, C=L + 5)
    qd, cache = q_to_dev(q), cache_to_dev(kc, ks, vc, vs)
    ref_o, ref_l = qkv.decode(qd, cache, L, num_splits=ns, return_lse=True)
    got_o, got_l = qkv.decode_noalloc(qd, cache, L, num_splits=ns, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(got_o, ref_o), f"{shape}: out differs from qkv_decode"
    assert torch.equal(got_l, ref_l), f"{shape}: lse differs from qkv_decode"
    ro, _ = oracle.attention(q, kc, ks, vc, vs, L, 1.0 / D ** 0.5)
    assert_close(got_o, ro, f"{shape} vs oracle")


def test_noalloc_two_calls_then_repeat():
    print("noalloc: shapes", SHAPES, flush=True)
    assert qkv.decode_auto_splits(*SHAPES[0][:6]) > 1   # the scratch is used
    _run(SHAPES[0], 1)
    _run(SHAPES[1], 2)
    _run(SHAPES[0], 3)


def test_noalloc_rejects_sizes_past_the_scratch():
    B, Hq, Hkv, Sq, L, D = 16, 64, 1, 1, 131072, 128
    qd = torch.zeros((B, Hq, Sq, D), dtype=torch.bfloat16, device=DEV)
    cache = qkv.KVCache(torch.zeros((B, Hkv, L, D // 2), dtype=torch.uint8, device=DEV),
                        torch.zeros((B, Hkv, L), dtype=torch.float16, device=DEV),
                        torch.zeros((B, Hkv, L, D // 2), dtype=torch.uint8, device=DEV),
                        torch.zeros((B, Hkv, L), dtype=torch.float16, device=DEV))
    with pytest.raises(Exception, match="static scratch"):
        qkv.decode_noalloc(qd, cache, L, num_splits=64)   # 1024 rows x 64 splits x 516 B > 16 MiB

"""GPU parity of the INT8 decode buffer: universal scale and flush byte for
byte against the oracle, decode over int4 rows + buffered rows against the
fp64 oracle, and a whole buffer life cycle (steps, flush, steps)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_flashattention_amd as qkv
from gpu_helpers import DEV, assert_close, cache_to_dev, compare, q_to_dev, random_case

pytestmark = pytest.mark.gpu


def _scales_np(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _buf_to_dev(kb, vb, k8, v8, length):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return qkv.DecodeBuffer(t(kb), t(vb), t(k8), t(v8), length)


@pytest.mark.parametrize("L", [0, 1, 100, 300])
def test_buffer_scale_matches_oracle(L):
    rng = np.random.default_rng(L)
    B, H, C = 3, 4, 300
    ks = rng.integers(0, 0x7800, size=(B, H, C), dtype=np.uint16)
    vs = rng.integers(0, 0x7800, size=(B, H, C), dtype=np.uint16)
    ks[0, 0] = 0                       # an all-zero row range
    vs[1, 2, : max(L - 1, 0)] = 0      # only the last row counts
    kc = np.zeros((B, H, C, 32), np.uint8)
    cache = cache_to_dev(kc, ks, kc, vs)
    buf = qkv.DecodeBuffer.empty(B, H, 64, device=DEV)
    buf.k_s8.fill_(-1.0)
    buf.v_s8.fill_(-1.0)
    qkv.buffer_scale(cache, L, buf)
    torch.cuda.synchronize()
    assert np.array_equal(buf.k_s8.cpu().numpy(), oracle.buffer_scale(ks, L))
    assert np.array_equal(buf.v_s8.cpu().numpy(), oracle.buffer_scale(vs, L))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T,pos", [(1, 0), (37, 5), (64, 200)])
def test_buffer_flush_matches_oracle(D, T, pos):
    rng = np.random.default_rng(T + D)
    B, H, rows, C = 2, 3, 64, 300
    kb = rng.integers(-127, 128, size=(B, H, rows, D), dtype=np.int8)
    vb = rng.integers(-127, 128, size=(B, H, rows, D), dtype=np.int8)
    kb[0, 0, :T] = 0                                           # all-zero rows
    vb[1, 1, :T, 0] = 127                                      # range ends
    k8 = rng.uniform(1e-3, 1.0, size=(B, H)).astype(np.float32)
    v8 = rng.uniform(1e-3, 1.0, size=(B, H)).astype(np.float32)
    k8[1, 2] = 0.0                                             # zero scale: zero rows
    v8[0, 1] = np.float32(2.0 ** -20)                          # tiny values
    buf = _buf_to_dev(kb, vb, k8, v8, T)
    cache = qkv.KVCache(*(torch.full(s, f, dtype=dt, device=DEV) for s, f, dt in (
        ((B, H, C, D // 2), 0xA5, torch.uint8), ((B, H, C), 1.5, torch.float16),
        ((B, H, C, D // 2), 0x5A, torch.uint8), ((B, H, C), -2.5, torch.float16))))
    qkv.buffer_flush(buf, cache, pos)
    torch.cuda.synchronize()
    assert buf.length == 0
    for codes, scales, src, s8, fc, fs in ((cache.k_codes, cache.k_scales, kb, k8, 0xA5, 1.5),
                                           (cache.v_codes, cache.v_scales, vb, v8, 0x5A, -2.5)):
        rc, rs = oracle.flush_rows(src[:, :, :T], s8)
        c, s = codes.cpu().numpy(), _scales_np(scales)
        assert np.array_equal(c[:, :, pos:pos + T], rc) and np.array_equal(s[:, :, pos:pos + T], rs)
        assert np.all(c[:, :, :pos] == fc) and np.all(c[:, :, pos + T:] == fc)
        f16 = np.float16(fs).view(np.uint16)
        assert np.all(s[:, :, :pos] == f16) and np.all(s[:, :, pos + T:] == f16)


def _buffered_case(seed, B, Hq, Hkv, Sq, L, C, buf_len, n_new, D):
    q, kc, ks, vc, vs = random_case(seed, B, Hq, Hkv, Sq, max(L, 1), D, C)
    rng = np.random.default_rng(seed + 7)
    k8 = oracle.buffer_scale(ks, L) if L > 0 else rng.uniform(0.01, 0.03, size=(B, Hkv)).astype(np.float32)
    v8 = oracle.buffer_scale(vs, L) if L > 0 else rng.uniform(0.01, 0.03, size=(B, Hkv)).astype(np.float32)
    kb = rng.integers(-127, 128, size=(B, Hkv, 64, D), dtype=np.int8)    # rows >= buf_len: garbage
    vb = rng.integers(-127, 128, size=(B, Hkv, 64, D), dtype=np.int8)
    k_new = rng.standard_normal((B, Hkv, n_new, D)).astype(np.float32)
    v_new = rng.standard_normal((B, Hkv, n_new, D)).astype(np.float32)
    if n_new:
        k_new[0, 0, 0, :4] *= 40.0        # outliers past the universal range: clamped
        v_new[-1, -1, -1, 3] = -1e4
    return q, (kc, ks, vc, vs), (kb, vb, k8, v8), (k_new, v_new)


BUF_CASES = [
    # B, Hq, Hkv, Sq, L, C, buf_len, n_new, D, num_splits
    (2, 32, 8, 1, 1000, 1024, 10, 1, 128, 0),
    (1, 64, 8, 1, 4096, 4100, 63, 1, 128, 0),   # the step that fills the buffer
    (2, 8, 2, 4, 777, 800, 0, 1, 64, 3),         # first row of an empty buffer
    (1, 8, 2, 2, 300, 300, 20, 0, 128, 1),       # attend only
    (1, 4, 4, 1, 0, 8, 5, 3, 64, 0),             # no int4 rows: the buffer split alone
    (1, 4, 1, 16, 200, 256, 40, 24, 128, 0),     # 64 query rows per group, a full buffer
    (3, 12, 4, 1, 2049, 2100, 31, 2, 128, 5),
    (1, 8, 2, 1, 3000, 3100, 17, 1, 128, 8),     # 7 cache splits (interleaved) + the buffer split
    (1, 8, 2, 1, 3000, 3100, 17, 1, 128, 9),     # 8 cache splits (ranges) + the buffer split
]


@pytest.mark.parametrize("case", BUF_CASES, ids=[str(c) for c in BUF_CASES])
def test_decode_buffered_matches_oracle(case):
    B, Hq, Hkv, Sq, L, C, buf_len, n_new, D, ns = case
    q, cache, (kb, vb, k8, v8), (k_new, v_new) = _buffered_case(sum(case), B, Hq, Hkv, Sq, L, C, buf_len, n_new, D)
    buf = _buf_to_dev(kb, vb, k8, v8, buf_len)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    kw = {}
    if n_new:
        kw = dict(k_new=torch.from_numpy(k_new).to(DEV), v_new=torch.from_numpy(v_new).to(DEV))
    out, lse = qkv.decode_buffered(q_to_dev(q), cache_to_dev(*cache), L, buf, softmax_scale=scale, num_splits=ns,
                                   return_lse=True, **kw)
    torch.cuda.synchronize()
    assert buf.length == buf_len + n_new
    T = buf_len + n_new
    ekb, evb = kb.copy(), vb.copy()
    ekb[:, :, buf_len:T] = oracle.quantize_int8(k_new, k8[:, :, None])
    evb[:, :, buf_len:T] = oracle.quantize_int8(v_new, v8[:, :, None])
    assert np.array_equal(buf.k.cpu().numpy(), ekb), "K buffer rows differ"
    assert np.array_equal(buf.v.cpu().numpy(), evb), "V buffer rows differ"
    ro, rl = oracle.attention_buffered(q, *cache, L, ekb, evb, k8, v8, T, scale)
    assert_close(out, ro, f"buffered {case}")
    assert compare(lse, rl)[0] < 1e-3


def test_decode_buffered_without_rows_is_decode():
    """An empty buffer and no new rows: the plain decode, bit for bit."""
    B, Hq, Hkv, L, C, D = 2, 32, 8, 3000, 3100, 128
    q, kc, ks, vc, vs = random_case(3, B, Hq, Hkv, 1, L, D, C)
    cache = cache_to_dev(kc, ks, vc, vs)
    buf = qkv.DecodeBuffer.empty(B, Hkv, D, device=DEV)
    o1, l1 = qkv.decode_buffered(q_to_dev(q), cache, L, buf, softmax_scale=0.09, return_lse=True)
    o2, l2 = qkv.decode(q_to_dev(q), cache, L, softmax_scale=0.09, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_buffer_life_cycle():
    """70 one-token steps from a 500-row cache: the buffer fills (64 steps),
    is flushed into the cache (scales recomputed), and fills again.  Every step
    matches the oracle run through the same life cycle; the final cache and
    buffer match byte for byte."""
    B, Hq, Hkv, D, C, L0 = 2, 8, 2, 128, 700, 500
    q, kc, ks, vc, vs = random_case(9, B, Hq, Hkv, 1, L0, D, C)
    qd = q_to_dev(q)
    cache = cache_to_dev(kc, ks, vc, vs)
    buf = qkv.DecodeBuffer.empty(B, Hkv, D, device=DEV)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    rkc, rks, rvc, rvs = kc.copy(), ks.copy(), vc.copy(), vs.copy()
    rkb = np.zeros((B, Hkv, 64, D), np.int8)
    rvb = np.zeros((B, Hkv, 64, D), np.int8)
    L, T = L0, 0
    qkv.buffer_scale(cache, L, buf)
    rk8, rv8 = oracle.buffer_scale(rks, L), oracle.buffer_scale(rvs, L)
    rng = np.random.default_rng(4)
    for step in range(70):
        if T == 64:
            qkv.buffer_flush(buf, cache, L)
            fk, fks = oracle.flush_rows(rkb, rk8)
            fv, fvs = oracle.flush_rows(rvb, rv8)
            rkc[:, :, L:L + 64], rks[:, :, L:L + 64] = fk, fks
            rvc[:, :, L:L + 64], rvs[:, :, L:L + 64] = fv, fvs
            L, T = L + 64, 0
            qkv.buffer_scale(cache, L, buf)
            rk8, rv8 = oracle.buffer_scale(rks, L), oracle.buffer_scale(rvs, L)
        k_new = (rng.standard_normal((B, Hkv, 1, D)) * (1 + step / 20)).astype(np.float32)   # growing range
        v_new = rng.standard_normal((B, Hkv, 1, D)).astype(np.float32)
        out = qkv.decode_buffered(qd, cache, L, buf, torch.from_numpy(k_new).to(DEV), torch.from_numpy(v_new).to(DEV),
                                  softmax_scale=0.088, num_splits=3, workspace=ws)
        rkb[:, :, T] = oracle.quantize_int8(k_new[:, :, 0], rk8)
        rvb[:, :, T] = oracle.quantize_int8(v_new[:, :, 0], rv8)
        T += 1
        torch.cuda.synchronize()
        assert buf.length == T
        assert int((ws[:64] != 0).sum()) == 0, f"step {step}: tickets not returned to zero"
        if step % 7 == 0 or step in (63, 64, 69):
            ro, _ = oracle.attention_buffered(q, rkc, rks, rvc, rvs, L, rkb, rvb, rk8, rv8, T, 0.088)
            assert_close(out, ro, f"step {step}")
    assert np.array_equal(cache.k_codes.cpu().numpy(), rkc) and np.array_equal(_scales_np(cache.v_scales), rvs)
    assert np.array_equal(buf.k[:, :, :T].cpu().numpy(), rkb[:, :, :T])
    assert np.array_equal(buf.v_s8.cpu().numpy(), rv8)

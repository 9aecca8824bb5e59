"""GPU split-K decode parity against the fp64 oracle (max-abs 4e-3, mean-abs 4e-4).

The GPU consumes oracle-quantized caches (uploaded), so attention parity does
not depend on the GPU quantizer.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_flashattention_amd as qkv
from qkv_inputs import f32_to_bf16_bits
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
    (1, 2, 1, 1, 40000, 40000, 64),  # with 8 splits, ranges of 5024 tokens: scales not staged
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
@pytest.mark.parametrize("ns", [0, 1, 3, 8])
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


def test_workspace_reuse_across_shapes():
    """One zeroed workspace serves a sequence of calls with the same B*Hkv whose
    split counts and sizes change: the tickets sit at a fixed offset and each
    call leaves them at zero."""
    ws = torch.zeros(4 << 20, dtype=torch.uint8, device=DEV)
    for Sq, L, ns in [(4, 3000, 20), (1, 500, 2), (16, 999, 7), (2, 64, 2), (1, 4000, 0), (3, 3000, 20)]:
        q, kc, ks, vc, vs = random_case(L + Sq, 1, 8, 2, Sq, L, 128)
        out = qkv.decode(q_to_dev(q), cache_to_dev(kc, ks, vc, vs), L, softmax_scale=0.1, num_splits=ns,
                         workspace=ws)
        torch.cuda.synchronize()
        ro, _ = oracle.attention(q, kc, ks, vc, vs, L, 0.1)
        assert_close(out, ro, f"Sq={Sq} L={L} ns={ns}")
        assert int((ws[:8] != 0).sum()) == 0, "tickets not returned to zero"


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, Sq, L, D, num_splits
    (1, 1, 1, 1, 20000, 64, 200),     # one query row, 157 splits: 16 threads per output item
    (1, 2, 1, 1, 20000, 128, 200),    # 8 threads per item, more than 16 splits each
    (2, 4, 2, 3, 9000, 128, 40),      # 2 threads per item, 18 splits each
    (1, 8, 2, 8, 5000, 128, 40),      # 32 rows: one thread per item, loads in rounds
])
def test_merge_of_many_splits(case):
    """The merging workgroup spreads each output item's splits over several
    threads when there are few rows and many splits; every split's partial
    still counts once, and repeated calls agree bit for bit."""
    B, Hq, Hkv, Sq, L, D, ns = case
    q, kc, ks, vc, vs = random_case(sum(case), B, Hq, Hkv, Sq, L, D)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse = _run(q, (kc, ks, vc, vs), L, scale, ns)
    again, _ = _run(q, (kc, ks, vc, vs), L, scale, ns)
    assert torch.equal(out, again)
    ro, rl = oracle.attention(q, kc, ks, vc, vs, L, scale)
    assert_close(out, ro, f"{case}")
    assert compare(lse, rl)[0] < 1e-3


@pytest.mark.parametrize("case", [(16, 32, 8, 1, 8192, 128, 0), (1, 64, 8, 1, 20000, 128, 0), (2, 8, 2, 4, 3000, 64, 11)])
def test_split_merge_sees_fresh_partials(case):
    """The last workgroup of a group merges partials written by workgroups on
    other XCDs.  Alternate two caches of the same shape many times: every
    output must equal the first output of its own inputs bit for bit (a stale
    partial from the other input set would show up as a difference)."""
    B, Hq, Hkv, Sq, L, D, ns = case
    inputs = [random_case(100 + t, B, Hq, Hkv, Sq, L, D) for t in range(2)]
    dev = [(q_to_dev(q), cache_to_dev(kc, ks, vc, vs)) for q, kc, ks, vc, vs in inputs]
    first = [None, None]
    for it in range(24):
        t = it % 2
        out = qkv.decode(dev[t][0], dev[t][1], L, softmax_scale=0.09, num_splits=ns)
        torch.cuda.synchronize()
        if first[t] is None:
            first[t] = out.clone()
            q, kc, ks, vc, vs = inputs[t]
            heads = [(b, h) for b in range(min(B, 2)) for h in range(Hq)]
            ro, _ = oracle.attention(q, kc, ks, vc, vs, L, 0.09, heads=heads)
            assert_close(out, ro, f"{case} input {t}")
        else:
            assert torch.equal(out, first[t]), f"{case}: iteration {it} differs"


APPEND_CASES = [
    # B, Hq, Hkv, Sq, pos, n_new, C, D, num_splits
    (2, 8, 2, 1, 999, 1, 1024, 128, 0),
    (1, 64, 8, 1, 4096, 1, 4100, 128, 0),
    (2, 32, 8, 2, 777, 2, 800, 128, 3),
    (1, 8, 2, 5, 124, 5, 129, 64, 0),
    (1, 4, 1, 16, 300, 16, 320, 128, 0),    # 64 rows per group: the four-wave variant
    (1, 8, 2, 4, 1534, 4, 2048, 128, 4),    # new rows straddle the split boundary at 1536
    (1, 4, 2, 3, 0, 3, 8, 64, 0),           # the whole cache is new
    (1, 2, 2, 64, 100, 64, 200, 64, 0),     # the most new rows one call takes
    (3, 12, 4, 1, 2049, 2, 2100, 128, 0),   # two new rows, one query row
    (1, 8, 2, 1, 100, 64, 200, 64, 2),      # new rows in chunks 3, 4, 5: splits 1, 0, 1
    (2, 8, 2, 2, 60, 40, 128, 128, 3),      # new rows in chunks 1, 2, 3: splits 1, 2, 0
    (2, 6, 3, 1, 1499, 1, 1600, 128, 0),    # 2 rows per group (packed softmax), D 128
    (2, 3, 1, 1, 700, 2, 720, 64, 3),       # 3 rows per group (packed softmax), D 64
    (1, 2, 2, 2, 257, 3, 300, 64, 0),       # 2 rows per group from 2 query positions
    (1, 8, 2, 1, 2000, 1, 2100, 128, 8),    # 8 splits: each reads one range of chunks
    (2, 16, 2, 2, 777, 2, 800, 64, 12),     # ranges of 3 chunks, the last one ragged
    (1, 64, 8, 1, 8191, 1, 8192, 128, 32),  # 8 rows per group, 32 splits of 8 chunks
]


def _new_rows(seed, B, Hkv, n, D):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, Hkv, n, D)).astype(np.float32)
    v = (rng.standard_normal((B, Hkv, n, D)) * 2).astype(np.float32)
    k[0, 0, 0, :3] = 0.0      # exact zeros and a row with a large channel
    v[-1, -1, -1, 5] *= 9.0
    return k, v


@pytest.mark.parametrize("case", APPEND_CASES, ids=[str(c) for c in APPEND_CASES])
def test_decode_append_equals_append_then_decode(case):
    """The one-launch step writes the same cache rows and gives bit-identical
    out and lse as quantize_append_kv followed by decode; both match the oracle."""
    B, Hq, Hkv, Sq, pos, n_new, C, D, ns = case
    q, kc, ks, vc, vs = random_case(sum(case), B, Hq, Hkv, Sq, max(pos, 1), D, C)
    k_new, v_new = _new_rows(sum(case) + 1, B, Hkv, n_new, D)
    kn, vn = torch.from_numpy(k_new).to(DEV), torch.from_numpy(v_new).to(DEV)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    sep = cache_to_dev(kc, ks, vc, vs)
    fused = cache_to_dev(kc, ks, vc, vs)
    qkv.quantize_append_kv(kn, vn, sep, pos)
    o1, l1 = qkv.decode(q_to_dev(q), sep, pos + n_new, softmax_scale=scale, num_splits=ns, return_lse=True)
    o2, l2 = qkv.decode_append(q_to_dev(q), kn, vn, fused, pos, softmax_scale=scale, num_splits=ns,
                               return_lse=True)
    torch.cuda.synchronize()
    for a, b in zip(sep.tensors(), fused.tensors()):
        assert torch.equal(a, b), "cache rows differ"
    assert torch.equal(o1, o2), f"out differs: {float((o1 - o2).abs().max())}"
    assert torch.equal(l1, l2)
    rkc, rks = oracle.quantize_rows(k_new)
    rvc, rvs = oracle.quantize_rows(v_new)
    kc2, ks2, vc2, vs2 = kc.copy(), ks.copy(), vc.copy(), vs.copy()
    kc2[:, :, pos:pos + n_new], ks2[:, :, pos:pos + n_new] = rkc, rks
    vc2[:, :, pos:pos + n_new], vs2[:, :, pos:pos + n_new] = rvc, rvs
    assert np.array_equal(fused.k_codes.cpu().numpy(), kc2)
    assert np.array_equal(fused.v_scales.view(torch.int16).cpu().numpy().view(np.uint16), vs2)
    ro, rl = oracle.attention(q, kc2, ks2, vc2, vs2, pos + n_new, scale)
    assert_close(o2, ro, f"decode_append {case}")
    assert compare(l2, rl)[0] < 1e-3


def test_decode_append_steps_reuse_workspace():
    """Ten consecutive one-token steps on one cache and one workspace, each
    checked bit for bit against the two-launch step on a twin cache."""
    B, Hq, Hkv, D, C, L0 = 2, 16, 4, 128, 3100, 3000
    q, kc, ks, vc, vs = random_case(11, B, Hq, Hkv, 1, L0, D, C)
    qd = q_to_dev(q)
    sep, fused = cache_to_dev(kc, ks, vc, vs), cache_to_dev(kc, ks, vc, vs)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    for step in range(10):
        kn, vn = (torch.from_numpy(t).to(DEV) for t in _new_rows(100 + step, B, Hkv, 1, D))
        pos = L0 + step
        qkv.quantize_append_kv(kn, vn, sep, pos)
        o1 = qkv.decode(qd, sep, pos + 1, softmax_scale=0.09, num_splits=7)
        o2 = qkv.decode_append(qd, kn, vn, fused, pos, softmax_scale=0.09, num_splits=7, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), f"step {step}"
        assert int((ws[:64] != 0).sum()) == 0, "tickets not returned to zero"
    for a, b in zip(sep.tensors(), fused.tensors()):
        assert torch.equal(a, b)


@pytest.mark.parametrize("Hq,Hkv,Sq", [(3, 1, 1), (2, 1, 2), (1, 1, 3), (4, 2, 2), (6, 2, 1), (5, 1, 1)])
@pytest.mark.parametrize("ns", [0, 3])
def test_row_counts_around_packed_softmax(Hq, Hkv, Sq, ns):
    """Groups of 1-5 query rows (G x Sq): up to 4 rows the softmax runs on
    scores packed two per lane, 5 rows use the unpacked path."""
    B, L, D = 2, 1500, 128
    q, kc, ks, vc, vs = random_case(Hq * 10 + Hkv + Sq, B, Hq, Hkv, Sq, L, D)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse = _run(q, (kc, ks, vc, vs), L, scale, ns)
    ro, rl = oracle.attention(q, kc, ks, vc, vs, L, scale)
    assert_close(out, ro, f"Hq={Hq} Hkv={Hkv} Sq={Sq} ns={ns}")
    assert compare(lse, rl)[0] < 1e-3


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("Hq,Hkv,Sq", [(2, 1, 1), (6, 2, 1), (1, 1, 2), (1, 1, 3),
                                        (5, 1, 1), (3, 1, 2), (7, 1, 1), (8, 1, 1)])
def test_packed_softmax_across_widths(D, bits, Hq, Hkv, Sq):
    """Groups of 2, 3 (the 4-row packed softmax's partly filled lane groups)
    and 5-8 query rows (the 8-row packed form) at both head dims and every
    code width, with outlier channels in K and V, against the oracle (b-bit
    caches: the oracle's b-bit attention)."""
    B, L, C = 2, 1100, 1130
    seed = 31 * D + 7 * bits + 3 * Hq + Hkv + Sq
    scale = float(np.float32(1.0 / np.sqrt(D)))
    if bits == 4:
        q, kc, ks, vc, vs = random_case(seed, B, Hq, Hkv, Sq, L, D, C, outliers=True)
        out, lse = _run(q, (kc, ks, vc, vs), L, scale)
        ro, rl = oracle.attention(q, kc, ks, vc, vs, L, scale)
    else:
        rng = np.random.default_rng(seed)
        q = f32_to_bf16_bits(rng.standard_normal((B, Hq, Sq, D)).astype(np.float32))
        arrs = []
        for f in (1.0, 1.5):
            x = (rng.standard_normal((B, Hkv, C, D)) * f).astype(np.float32)
            x[:, :, :, rng.choice(D, size=2, replace=False)] *= 8.0     # outlier channels
            arrs += list(oracle.quantize_rows_bits(x, bits))
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
        h = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).to(DEV)
        cache = qkv.KVCache(t(arrs[0]), h(arrs[1]), t(arrs[2]), h(arrs[3]))
        out, lse = qkv.decode(q_to_dev(q), cache, L, softmax_scale=scale, return_lse=True, bits=bits)
        torch.cuda.synchronize()
        ro, rl = oracle.attention_bits(q, *arrs, L, scale, bits)
    assert_close(out, ro, f"D={D} bits={bits} rows={Hq // Hkv * Sq}")
    assert compare(lse, rl)[0] < 1e-3

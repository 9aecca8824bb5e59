"""GPU parity of the ragged / paged decode step (qkv_decode_paged).

Sequences of one batch hold different numbers of cached rows; with a block
table their rows are scattered over a shared page pool in shuffled order.
Each sequence is checked against the fp64 oracle run on its own rows alone
(gathered from the pool on the host), appended rows byte for byte against the
oracle quantizer, and every other pool row must be left as it was.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_flashattention_amd as qkv
from gpu_helpers import DEV, assert_close, compare, q_to_dev
from qkv_inputs import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _ceil(a, b):
    return -(-a // b)


def _pool_case(seed, B, Hq, Hkv, Sq, lens, D, P, n_new, paged, extra_pages=3):
    """Random queries, new rows and a pool holding every sequence's cached rows.

    paged: pages of P rows in shuffled order, addressed through a block table
    whose unused entries hold out-of-range junk; else one entry of capacity P
    per sequence (the contiguous layout, no table).
    """
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, Sq, D)).astype(np.float32))
    if paged:
        max_pages = max(1, _ceil(max(lens) + n_new, P))
        used = [_ceil(L + n_new, P) for L in lens]
        num_pages = sum(used) + extra_pages
        perm = rng.permutation(num_pages).astype(np.int32)
        table = rng.choice(np.array([-1, -7, num_pages, 1 << 30], np.int32), size=(B, max_pages))
        k = 0
        for b in range(B):
            table[b, :used[b]] = perm[k:k + used[b]]
            k += used[b]
    else:
        num_pages, table = B + extra_pages, None
    pool = [rng.integers(0, 256, size=(num_pages, Hkv, P, D // 2), dtype=np.uint8),
            rng.integers(0, 0x7800, size=(num_pages, Hkv, P), dtype=np.uint16),
            rng.integers(0, 256, size=(num_pages, Hkv, P, D // 2), dtype=np.uint8),
            rng.integers(0, 0x7800, size=(num_pages, Hkv, P), dtype=np.uint16)]
    for b, L in enumerate(lens):
        k_rows = rng.standard_normal((Hkv, L, D)).astype(np.float32)
        v_rows = (rng.standard_normal((Hkv, L, D)) * 1.5).astype(np.float32)
        kc, ks = oracle.quantize_rows(k_rows)
        vc, vs = oracle.quantize_rows(v_rows)
        _scatter(pool, table, b, 0, (kc, ks, vc, vs), P)
    k_new = rng.standard_normal((B, Hkv, n_new, D)).astype(np.float32)
    v_new = (rng.standard_normal((B, Hkv, n_new, D)) * 2).astype(np.float32)
    return q, pool, table, k_new, v_new


def _page(table, b, i):
    return b if table is None else int(table[b, i])


def _scatter(pool, table, b, t0, rows, P):
    """Write rows (codes/scales [Hkv, n, ...] x4) of sequence b from token t0 on."""
    n = rows[0].shape[1]
    t = t0
    while t < t0 + n:
        pg, r = _page(table, b, t // P), t % P
        m = min(P - r, t0 + n - t)
        for arr, src in zip(pool, rows):
            arr[pg, :, r:r + m] = src[:, t - t0:t - t0 + m]
        t += m


def _gather(pool, table, b, L, P):
    """Rows [0, L) of sequence b as a one-sequence contiguous cache [1, Hkv, L, ...]."""
    out = []
    for arr in pool:
        parts = [arr[_page(table, b, i), :, :min(P, L - i * P)] for i in range(_ceil(L, P))]
        cat = np.concatenate(parts, axis=1) if parts else arr[0, :, :0]
        out.append(cat[None])
    return out


def _to_dev(pool):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    h = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).to(DEV)
    return qkv.KVCache(t(pool[0]), h(pool[1]), t(pool[2]), h(pool[3]))


def _from_dev(cache):
    return [cache.k_codes.cpu().numpy(), cache.k_scales.view(torch.int16).cpu().numpy().view(np.uint16),
            cache.v_codes.cpu().numpy(), cache.v_scales.view(torch.int16).cpu().numpy().view(np.uint16)]


def _run(q, pool, table, lens, k_new, v_new, scale, ns=0, max_kv_len="tight", workspace=None):
    cache = _to_dev(pool)
    n_new = k_new.shape[2]
    kw = {}
    if n_new:
        kw = dict(k_new=torch.from_numpy(k_new).to(DEV), v_new=torch.from_numpy(v_new).to(DEV))
    bt = None if table is None else torch.from_numpy(table).to(DEV)
    kl = torch.tensor(np.asarray(lens, np.int32), device=DEV)
    mkl = max(max(lens) + n_new, 1) if max_kv_len == "tight" else max_kv_len
    out, lse = qkv.decode_paged(q_to_dev(q), cache, kl, bt, max_kv_len=mkl, softmax_scale=scale,
                                num_splits=ns, return_lse=True, workspace=workspace, **kw)
    torch.cuda.synchronize()
    return out, lse, cache


def _expected_pool(pool, table, lens, k_new, v_new, P):
    exp = [a.copy() for a in pool]
    if k_new.shape[2]:
        kc, ks = oracle.quantize_rows(k_new)
        vc, vs = oracle.quantize_rows(v_new)
        for b, L in enumerate(lens):
            _scatter(exp, table, b, L, (kc[b], ks[b], vc[b], vs[b]), P)
    return exp


def _check(q, exp_pool, table, lens, n_new, P, scale, out, lse, what):
    for b, L in enumerate(lens):
        Lb = L + n_new
        if Lb == 0:
            assert bool((out[b] == 0).all()), f"{what}: empty sequence {b} output not zero"
            assert bool(torch.isneginf(lse[b]).all()), f"{what}: empty sequence {b} lse not -inf"
            continue
        kc, ks, vc, vs = _gather(exp_pool, table, b, Lb, P)
        ro, rl = oracle.attention(q[b:b + 1], kc, ks, vc, vs, Lb, scale)
        assert_close(out[b:b + 1], ro, f"{what} seq {b} L={Lb}")
        assert compare(lse[b:b + 1], rl)[0] < 1e-3


CASES = [
    # B, Hq, Hkv, Sq, lens, D, P, n_new, num_splits
    (4, 8, 2, 1, (1, 31, 777, 2049), 128, 64, 0, 0),
    (3, 32, 8, 1, (4096, 100, 0), 128, 256, 0, 0),          # an empty sequence
    (2, 8, 2, 4, (129, 1000), 64, 32, 0, 3),
    (5, 16, 4, 1, (300, 301, 5000, 64, 65), 128, 128, 1, 0),
    (2, 32, 8, 1, (8191, 3), 128, 512, 1, 0),
    (1, 4, 1, 16, (700,), 128, 32, 16, 0),                   # 64 rows per group; new rows cross a page
    (3, 8, 2, 1, (0, 0, 40), 64, 32, 2, 5),                  # appends into empty sequences
    (2, 8, 8, 1, (20000, 17), 64, 32, 0, 1),                 # one split over 625 pages
    (4, 8, 2, 1, (50, 700, 2500, 9000), 128, 64, 1, 40),    # 2, 22, 40, 40 live splits: both merge forms
    (3, 6, 2, 1, (700, 1500, 33), 128, 64, 1, 0),            # 3 rows per group (packed softmax)
    (2, 4, 2, 1, (2000, 5), 64, 32, 1, 3),                   # 2 rows per group (packed softmax)
]


@pytest.mark.parametrize("paged", [True, False], ids=["paged", "contiguous"])
@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_paged_decode_matches_oracle(case, paged):
    B, Hq, Hkv, Sq, lens, D, P, n_new, ns = case
    if not paged:
        P = max(lens) + n_new + 5        # per-sequence capacity of the contiguous cache
    q, pool, table, k_new, v_new = _pool_case(sum(lens) + D + n_new, B, Hq, Hkv, Sq, lens, D, P, n_new, paged)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse, cache = _run(q, pool, table, lens, k_new, v_new, scale, ns)
    exp = _expected_pool(pool, table, lens, k_new, v_new, P)
    got = _from_dev(cache)
    for name, g, e in zip(("k codes", "k scales", "v codes", "v scales"), got, exp):
        assert np.array_equal(g, e), f"pool {name} differs from the expected rows"
    _check(q, exp, table, lens, n_new, P, scale, out, lse, f"{case} paged={paged}")


@pytest.mark.parametrize("n_new,ns", [(0, 1), (1, 1), (0, 0), (1, 0), (3, 4)])
def test_paged_equals_contiguous(n_new, ns):
    """Equal lengths and a tight bound.  With one split the paged step is the
    contiguous step bit for bit (same arithmetic, only the addresses differ);
    with several, a paged split takes a range of consecutive chunks and a
    contiguous one interleaved chunks, so the two agree up to the merge's
    rounding.  The cache rows an appending step writes are identical."""
    B, Hq, Hkv, D, P, L = 3, 32, 8, 128, 64, 3000
    lens = (L,) * B
    q, pool, table, k_new, v_new = _pool_case(5, B, Hq, Hkv, 1, lens, D, P, n_new, True)
    out, lse, cache = _run(q, pool, table, lens, k_new, v_new, 0.088, ns)
    cc = [np.stack([_gather(pool, table, b, L, P)[i][0] for b in range(B)]) for i in range(4)]
    C = L + n_new + 7
    full = [np.zeros((B, Hkv, C) + a.shape[3:], a.dtype) for a in cc]
    for f, a in zip(full, cc):
        f[:, :, :L] = a
    ref = _to_dev(full)
    if n_new:
        o2, l2 = qkv.decode_append(q_to_dev(q), torch.from_numpy(k_new).to(DEV), torch.from_numpy(v_new).to(DEV),
                                   ref, L, softmax_scale=0.088, num_splits=ns, return_lse=True)
    else:
        o2, l2 = qkv.decode(q_to_dev(q), ref, L, softmax_scale=0.088, num_splits=ns, return_lse=True)
    torch.cuda.synchronize()
    if ns == 1:
        assert torch.equal(out, o2), f"max diff {float((out - o2).abs().max())}"
        assert torch.equal(lse, l2)
    else:
        # each side rounds P~ = p s_V to fp16 once per value: an output moves by
        # at most 2^-11 * 7 * max s_V on either side (7 = the largest |code|)
        vs_max = float(np.concatenate([cc[3].reshape(-1).view(np.float16).astype(np.float32),
                                       np.abs(v_new).reshape(-1) / 7]).max())
        assert float((out - o2).abs().max()) <= 2 * 2.0 ** -11 * 7 * vs_max
        assert float((lse - l2).abs().max()) < 1e-5
    if n_new:
        got = _from_dev(cache)
        want = _from_dev(ref)
        for b in range(B):
            g = _gather(got, table, b, L + n_new, P)
            for i in range(4):
                assert np.array_equal(g[i][0], want[i][b, :, :L + n_new])


def test_paged_lengths_are_clamped():
    """kv_lens outside [0, max_kv_len - n_new] act as the nearest bound."""
    B, Hq, Hkv, D, P, n_new = 3, 8, 2, 64, 32, 1
    lens = (100, 0, 63)
    q, pool, table, k_new, v_new = _pool_case(77, B, Hq, Hkv, 1, lens, D, P, n_new, True)
    o1, l1, _ = _run(q, pool, table, lens, k_new, v_new, 0.125, max_kv_len=101)
    o2, l2, _ = _run(q, pool, table, (10 ** 6, -5, 63), k_new, v_new, 0.125, max_kv_len=101)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_default_bound_matches_oracle():
    """Without max_kv_len the plan covers the whole table width; splits past
    a sequence's end do nothing and the result is unchanged."""
    B, Hq, Hkv, D, P, n_new = 2, 16, 4, 128, 256, 1
    lens = (1500, 20)
    q, pool, table, k_new, v_new = _pool_case(3, B, Hq, Hkv, 1, lens, D, P, n_new, True, extra_pages=0)
    table_wide = np.concatenate([table, np.full((B, 30), -1, np.int32)], axis=1)   # 36 pages of room
    out, lse, cache = _run(q, pool, table_wide, lens, k_new, v_new, 0.1, max_kv_len=None)
    exp = _expected_pool(pool, table, lens, k_new, v_new, P)
    assert all(np.array_equal(g, e) for g, e in zip(_from_dev(cache), exp))
    _check(q, exp, table, lens, n_new, P, 0.1, out, lse, "default bound")


def test_paged_steps_reuse_workspace():
    """Eight one-token steps of a ragged batch on one pool and one workspace;
    every step matches the oracle and leaves the tickets at zero."""
    B, Hq, Hkv, D, P = 3, 8, 2, 128, 64
    lens0 = [500, 1, 1200]
    steps = 8
    q, pool, table, _, _ = _pool_case(21, B, Hq, Hkv, 1, lens0, D, P, steps, True)
    cache = _to_dev(pool)
    exp = [a.copy() for a in pool]
    bt = torch.from_numpy(table).to(DEV)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(8)
    for s in range(steps):
        lens = [L + s for L in lens0]
        k_new = rng.standard_normal((B, Hkv, 1, D)).astype(np.float32)
        v_new = rng.standard_normal((B, Hkv, 1, D)).astype(np.float32)
        out, lse = qkv.decode_paged(q_to_dev(q), cache, torch.tensor(lens, dtype=torch.int32, device=DEV), bt,
                                    torch.from_numpy(k_new).to(DEV), torch.from_numpy(v_new).to(DEV),
                                    max_kv_len=max(lens0) + steps, softmax_scale=0.09, num_splits=6,
                                    return_lse=True, workspace=ws)
        torch.cuda.synchronize()
        assert int((ws[:64] != 0).sum()) == 0, f"step {s}: tickets not returned to zero"
        exp = _expected_pool(exp, table, lens, k_new, v_new, P)
        _check(q, exp, table, lens, 1, P, 0.09, out, lse, f"step {s}")
    assert all(np.array_equal(g, e) for g, e in zip(_from_dev(cache), exp))

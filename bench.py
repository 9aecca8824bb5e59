"""Benchmark of the int4-KV attention hot path on one MI355X.

One step = one decode step of the Llama-3-8B shaped GQA decode workload
(B=16, 32 query / 8 KV heads, D=128, 8192 cached tokens): quantize-and-append
the new token's K and V rows, then split-K decode attention of the query over
the whole cache (exact int4 -> fp16 conversion, MFMA QK^T and PV, online
softmax, LSE merge) -- both in one launch (qkv_decode_append).  Inputs are resident in HBM
before timing starts; the cache is rotated over several independent copies
so that the 256 MB Infinity Cache cannot serve repeated reads.  Timed
launches are queued behind a GPU hold so that host-side Python launch
overhead is excluded (the GPU runs them back to back, as a captured graph
would).

Printed (stdout, one JSON line): the headline decode throughput in GB/s of
packed KV bytes (codes + scales) per step, the roofline of the decode kernel
(achieved HBM GB/s of its algorithmic bytes over its average launch duration
in the timed region -- one launch per step -- measured with HIP events on the
launch stream), the CPU oracle timed on a bounded sample of the same
workload (and of the ViT-B and 16K causal prefill workloads), and secondary
figures (128K-token decode, a ragged 64-sequence batch over a paged cache,
the decode step with the INT8 buffer, decode over 2- and 3-bit and
asymmetric caches, 16K causal prefill TFLOP/s, ViT-B prefill GB/s and
TFLOP/s, the achievable-HBM streaming read, bulk quantize-append).
Everything else goes to stderr.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only headline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "int4-KV decode GB/s (% of HBM peak); prefill attention TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, published
MALL_BYTES = 256 * 2 ** 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of what the decode kernel is built from (its source, the shared
    device header, the split planner's inputs and the compiler flags):
    counter-derived traffic is valid only for exactly these."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "quantized_kv_flashattention_amd")
    for rel in ("csrc/decode.hip", "csrc/qkvfa_device.hpp", "csrc/qkvfa_internal.h", "build.py"):
        with open(os.path.join(pkg, rel), "rb") as f:
            h.update(rel.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    missing or taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    e = t.get("kernels", {}).get(kernel_key)
    return None if e is None else e.get("bytes_per_launch")


def upload_cache(torch, qkv, k, v, n_copies):
    """Quantize fp32 K/V on the GPU into a cache, then clone it n_copies-1 times."""
    B, H, L, D = k.shape
    c0 = qkv.KVCache.empty(B, H, L, D)
    kt = torch.from_numpy(k).cuda()
    qkv.quantize_append(kt, c0.k_codes, c0.k_scales, 0)
    del kt
    vt = torch.from_numpy(v).cuda()
    qkv.quantize_append(vt, c0.v_codes, c0.v_scales, 0)
    del vt
    caches = [c0] + [qkv.KVCache(*(t.clone() for t in c0.tensors())) for _ in range(n_copies - 1)]
    torch.cuda.synchronize()
    return caches


_SLEEP_CYCLES_PER_MS = None


def hold_gpu(torch, ms):
    """Queue a GPU spin of about `ms` milliseconds on the current stream.

    Launches enqueued behind it pile up while it runs, so the timed kernels
    run back to back and the host's per-launch Python overhead (tens of us,
    comparable to a decode kernel) is not measured -- as with a captured
    graph.  The spin's rate is calibrated once with events."""
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        a.record()
        torch.cuda._sleep(2_000_000)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = 2_000_000 / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(_SLEEP_CYCLES_PER_MS * ms))


def host_enqueue_ms(fn, n):
    """Host time to enqueue n calls of fn (no synchronization)."""
    t0 = time.perf_counter()
    for i in range(n):
        fn(i)
    return (time.perf_counter() - t0) * 1e3


def region_ms(torch, fn, n, rotate):
    """Average duration of fn(i) over n back-to-back calls, bracketed by HIP
    events on the launch stream and queued behind a GPU hold."""
    enq = host_enqueue_ms(lambda i: fn(i % rotate), 4) / 4
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    hold_gpu(torch, 2.0 * enq * n + 1.0)
    e0.record()
    for i in range(n):
        fn(i % rotate)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def per_launch_ms(torch, fn, n, rotate):
    """Average duration of fn(i) measured with HIP events recorded around each
    launch on the launch stream, with the launches queued behind a GPU hold."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    enq = host_enqueue_ms(lambda i: fn(i % rotate), 4)
    torch.cuda.synchronize()
    hold_gpu(torch, 2.0 * enq / 4 * n + 1.0)
    for i in range(n):
        starts[i].record()
        fn(i % rotate)
        ends[i].record()
    torch.cuda.synchronize()
    t = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return sum(t) / len(t), t[len(t) // 2]


def decode_bytes(w):
    codes = 2 * w.B * w.Hkv * w.L * (w.D // 2)
    scales = 2 * w.B * w.Hkv * w.L * 2
    q = w.B * w.Hq * w.Sq * w.D * 2
    o = w.B * w.Hq * w.Sq * w.D * 4
    return codes + scales, codes + scales + q + o


def prefill_flops(w):
    pairs = w.Sq * (w.Sq + 1) // 2 if (w.causal and w.Sq == w.L) else (
        sum(min(w.L, i + w.L - w.Sq + 1) for i in range(w.Sq)) if w.causal else w.Sq * w.L)
    return 4.0 * w.D * pairs * w.B * w.Hq


def prefill_bytes(w, bits=4, group=0):
    """Algorithmic HBM bytes of a prefill: Q (bf16) and O (fp32) once, every
    KV head's cache rows [0, L) once (codes + scales or parameter words)."""
    row = w.D * bits // 8 + (4 * (w.D // group) if group else 2)
    return w.B * w.Hq * w.Sq * w.D * (2 + 4) + 2 * w.B * w.Hkv * w.L * row


def bench_decode(torch, qkv, w, steps, warmup, with_append):
    from qkv_inputs import make_qkv
    q_bits, k, v = make_qkv(w)
    kv_bytes, attn_bytes = decode_bytes(w)
    n_copies = max(4, math.ceil(2.5 * MALL_BYTES / kv_bytes))
    caches = upload_cache(torch, qkv, k, v, n_copies)
    k_new = torch.from_numpy(k[:, :, -1:].copy()).cuda()
    v_new = torch.from_numpy(v[:, :, -1:].copy()).cuda()
    del k, v
    q = torch.from_numpy(q_bits.view("int16")).cuda().view(torch.bfloat16)
    out = torch.empty((w.B, w.Hq, w.Sq, w.D), dtype=torch.float32, device="cuda")
    ns = qkv.decode_auto_splits(w.B, w.Hq, w.Hkv, w.Sq, w.L, w.D)
    ws_bytes = qkv.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.L, w.D)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")   # tickets start at zero

    def decode_only(i):
        qkv.decode(q, caches[i], w.L, softmax_scale=w.softmax_scale, out=out, workspace=ws)

    def step(i):
        if with_append:   # the new token's K and V rows go to row L-1, then decode: one launch
            qkv.decode_append(q, k_new, v_new, caches[i], w.L - 1, softmax_scale=w.softmax_scale, out=out,
                              workspace=ws)
        else:
            decode_only(i)

    for i in range(warmup):
        step(i % n_copies)
    torch.cuda.synchronize()
    enq = host_enqueue_ms(lambda i: step(i % n_copies), 4) / 4
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    hold_gpu(torch, 2.0 * enq * steps + 1.0)
    e0.record()
    for i in range(steps):
        step(i % n_copies)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    # the step's kernel, one launch at a time (events on the launch stream)
    avg_ms, med_ms = per_launch_ms(torch, step, max(steps, 20), n_copies)
    plain_avg, _ = per_launch_ms(torch, decode_only, max(steps, 20), n_copies)
    if with_append:   # + the new rows' fp32 K and V read by the kernel
        attn_bytes += 2 * w.B * w.Hkv * w.D * 4
    # A step is exactly one launch of the decode kernel, so the timed region's
    # average per step is that kernel's average launch duration (back to
    # back, as rocprofv3 times it).  Event pairs around single launches add
    # the events' own packet overhead (~2 us); reported alongside.
    res = {
        "workload": w.name, "n_split": ns, "cache_copies": n_copies,
        "ms_per_step": ms_step,
        "packed_kv_bytes": kv_bytes, "algorithmic_bytes": attn_bytes,
        "step_GBps_packed_kv": kv_bytes / (ms_step * 1e-3) / 1e9,
        "kernel_GBps": attn_bytes / (ms_step * 1e-3) / 1e9,
        "single_launch_avg_ms": avg_ms, "single_launch_median_ms": med_ms,
        "decode_only_single_launch_avg_ms": plain_avg,
    }
    res["kernel_frac_hbm"] = res["kernel_GBps"] / HBM_PEAK_GBS
    del caches
    torch.cuda.empty_cache()
    return res


def build_paged(torch, qkv, w, seed=0):
    """Page pool, table and lengths of a ragged paged workload, quantized on the GPU."""
    from qkv_inputs import pool_rows, ragged_layout
    lens, table, num_pages = ragged_layout(w, seed)
    P, half = w.page_size, w.D // 2
    pool = qkv.KVCache(torch.empty((num_pages, w.Hkv, P, half), dtype=torch.uint8, device="cuda"),
                       torch.empty((num_pages, w.Hkv, P), dtype=torch.float16, device="cuda"),
                       torch.empty((num_pages, w.Hkv, P, half), dtype=torch.uint8, device="cuda"),
                       torch.empty((num_pages, w.Hkv, P), dtype=torch.float16, device="cuda"))
    for p0, k, v in pool_rows(w, num_pages, 512, seed):
        n = k.shape[0]
        qkv.quantize_append(torch.from_numpy(k).cuda(), pool.k_codes[p0:p0 + n], pool.k_scales[p0:p0 + n], 0)
        qkv.quantize_append(torch.from_numpy(v).cuda(), pool.v_codes[p0:p0 + n], pool.v_scales[p0:p0 + n], 0)
    torch.cuda.synchronize()
    return lens, table, num_pages, pool


def paged_bytes(w, lens, num_used_pages):
    """Algorithmic bytes of one ragged paged step (append 1 token + decode)."""
    rows = int(lens.sum())
    kv = 2 * rows * w.Hkv * (w.D // 2 + 2)
    other = (w.B * w.Hq * w.Sq * w.D * 2 + w.B * w.Hq * w.Sq * w.D * 4   # q, out
             + 2 * w.B * w.Hkv * w.D * 4                                  # new K/V rows (fp32)
             + 4 * num_used_pages + 4 * w.B)                              # page ids, lengths
    return kv, kv + other


def bench_paged(torch, qkv, w, steps):
    """Ragged batch over a shared page pool: one step appends every sequence's
    new token and attends its own rows (qkv_decode_paged, one launch)."""
    from qkv_inputs import make_qkv
    lens, table, num_pages, pool = build_paged(torch, qkv, w)
    rng_w = w.scaled(L=1)        # q and the new rows only
    q_bits, k1, v1 = make_qkv(rng_w)
    q = torch.from_numpy(q_bits.view("int16")).cuda().view(torch.bfloat16)
    k_new, v_new = torch.from_numpy(k1).cuda(), torch.from_numpy(v1).cuda()
    bt = torch.from_numpy(table).cuda()
    cached = torch.from_numpy(lens - 1).cuda()        # rows before the step; the step appends one
    out = torch.empty((w.B, w.Hq, w.Sq, w.D), dtype=torch.float32, device="cuda")
    max_len = int(lens.max())
    # the library's plan for per-sequence lengths: its uniform plan, with splits of at most 128 chunks
    ns = max(qkv.decode_auto_splits(w.B, w.Hq, w.Hkv, w.Sq, max_len, w.D), -(-max_len // 4096))
    ws = torch.zeros(max(qkv.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, max_len, w.D), 1),
                     dtype=torch.uint8, device="cuda")

    def step(_):
        qkv.decode_paged(q, pool, cached, bt, k_new, v_new, max_kv_len=max_len, softmax_scale=w.softmax_scale,
                         out=out, workspace=ws)

    for i in range(5):
        step(i)
    torch.cuda.synchronize()
    avg_ms = region_ms(torch, step, steps, 1)
    kv_bytes, alg = paged_bytes(w, lens, num_pages)
    res = {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "page_size": w.page_size,
           "lengths": f"uniform in [{w.len_min}, {w.L}], sum {int(lens.sum())}", "n_split": ns,
           "packed_kv_bytes": kv_bytes, "algorithmic_bytes": alg,
           "avg_ms": avg_ms, "GBps": alg / (avg_ms * 1e-3) / 1e9}
    res["frac_hbm"] = res["GBps"] / HBM_PEAK_GBS
    del pool
    torch.cuda.empty_cache()
    return res


def bench_buffered(torch, qkv, w, steps, buf_len=31):
    """Decode step with the INT8 buffer: int4 rows [0, L - buf_len - 1), buf_len
    buffered rows, and the step's new row quantized into the buffer -- L rows
    attended in all, as in the headline step.  Also the flush of a full
    buffer (64 rows) into the int4 cache, which runs once every 64 steps."""
    from qkv_inputs import make_qkv
    q_bits, k, v = make_qkv(w)
    kv_bytes, _ = decode_bytes(w)
    n_copies = max(4, math.ceil(2.5 * MALL_BYTES / kv_bytes))
    caches = upload_cache(torch, qkv, k, v, n_copies)
    body = w.L - buf_len - 1
    rows = torch.from_numpy(k[:, :, body:].copy()).cuda(), torch.from_numpy(v[:, :, body:].copy()).cuda()
    del k, v
    q = torch.from_numpy(q_bits.view("int16")).cuda().view(torch.bfloat16)
    out = torch.empty((w.B, w.Hq, w.Sq, w.D), dtype=torch.float32, device="cuda")
    bufs = []
    for c in caches:
        b = qkv.DecodeBuffer.empty(w.B, w.Hkv, w.D, device="cuda")
        qkv.buffer_scale(c, body, b)
        qkv.decode_buffered(q, c, body, b, rows[0][:, :, :buf_len].contiguous(), rows[1][:, :, :buf_len].contiguous(),
                            out=out)
        bufs.append(b)
    k_new, v_new = rows[0][:, :, buf_len:].contiguous(), rows[1][:, :, buf_len:].contiguous()
    ws = torch.zeros(max(qkv.decode_buffered_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, body, w.D), 1),
                     dtype=torch.uint8, device="cuda")

    def step(i):
        bufs[i].length = buf_len          # every timed step appends the same row
        qkv.decode_buffered(q, caches[i], body, bufs[i], k_new, v_new, softmax_scale=w.softmax_scale, out=out,
                            workspace=ws)

    for i in range(5):
        step(i % n_copies)
    torch.cuda.synchronize()
    ms = region_ms(torch, step, steps, n_copies)
    # flush of a full buffer (64 rows) into int4 cache rows
    full = qkv.DecodeBuffer.empty(w.B, w.Hkv, w.D, device="cuda")
    full.k.random_(-127, 128)
    full.v.random_(-127, 128)
    full.k_s8.fill_(0.02)
    full.v_s8.fill_(0.02)

    def flush(i):
        full.length = 64
        qkv.buffer_flush(full, caches[i], 0)

    for i in range(3):
        flush(i % n_copies)
    flush_ms = region_ms(torch, flush, 20, n_copies)
    int4 = 2 * w.B * w.Hkv * body * (w.D // 2 + 2)
    buffered = 2 * w.B * w.Hkv * (buf_len + 1) * w.D + 2 * w.B * w.Hkv * 4
    other = w.B * w.Hq * w.Sq * w.D * 6 + 2 * w.B * w.Hkv * w.D * 4
    res = {"workload": w.name + "+int8_buffer", "int4_rows": body, "buffered_rows": buf_len + 1,
           "step_ms": ms, "algorithmic_bytes": int4 + buffered + other,
           "GBps": (int4 + buffered + other) / (ms * 1e-3) / 1e9,
           "flush_64_rows_ms": flush_ms, "flush_ms_per_step": flush_ms / 64}
    res["frac_hbm"] = res["GBps"] / HBM_PEAK_GBS
    del caches, bufs
    torch.cuda.empty_cache()
    return res


def bench_lowbit(torch, qkv, w, steps):
    """Decode over 2-, 3- and 4-bit caches of the same workload (decode only,
    timed region of back-to-back launches, caches rotated past the MALL)."""
    from qkv_inputs import make_qkv
    q_bits, k, v = make_qkv(w)
    q = torch.from_numpy(q_bits.view("int16")).cuda().view(torch.bfloat16)
    out = torch.empty((w.B, w.Hq, w.Sq, w.D), dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(qkv.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.L, w.D), 1), dtype=torch.uint8,
                     device="cuda")
    kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    del k, v
    res = {"workload": w.name, "n_split": qkv.decode_auto_splits(w.B, w.Hq, w.Hkv, w.Sq, w.L, w.D)}
    for bits in (4, 3, 2):
        kv_bytes = 2 * w.B * w.Hkv * w.L * (w.D * bits // 8 + 2)
        n_copies = max(4, math.ceil(2.5 * MALL_BYTES / kv_bytes))
        c0 = qkv.KVCache.empty(w.B, w.Hkv, w.L, w.D, bits=bits)
        qkv.quantize_append_kv(kt, vt, c0, 0, bits=bits)
        caches = [c0] + [qkv.KVCache(*(t.clone() for t in c0.tensors())) for _ in range(n_copies - 1)]

        def run(i):
            qkv.decode(q, caches[i], w.L, softmax_scale=w.softmax_scale, out=out, workspace=ws, bits=bits)

        for i in range(5):
            run(i % n_copies)
        torch.cuda.synchronize()
        ms = region_ms(torch, run, steps, n_copies)
        alg = kv_bytes + w.B * w.Hq * w.Sq * w.D * 6
        res[f"{bits}bit"] = {"ms": ms, "kv_bytes": kv_bytes, "GBps": alg / (ms * 1e-3) / 1e9,
                             "frac_hbm": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del caches, c0
        torch.cuda.empty_cache()
    for bits in (3, 2):
        res[f"{bits}bit"]["speedup_vs_4bit"] = res["4bit"]["ms"] / res[f"{bits}bit"]["ms"]
    return res


def bench_asym(torch, qkv, w, steps, int4_ms=None):
    """Decode over asymmetric group-wise int4 caches of the same workload (groups
    of 32, 64 and 128 elements; decode only, caches rotated past the MALL)."""
    from qkv_inputs import make_qkv
    q_bits, k, v = make_qkv(w)
    q = torch.from_numpy(q_bits.view("int16")).cuda().view(torch.bfloat16)
    out = torch.empty((w.B, w.Hq, w.Sq, w.D), dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(qkv.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.L, w.D), 1), dtype=torch.uint8,
                     device="cuda")
    kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    del k, v
    res = {"workload": w.name}
    for group in (32, 64, 128):
        kv_bytes = 2 * w.B * w.Hkv * w.L * (w.D // 2 + 4 * (w.D // group))
        n_copies = max(4, math.ceil(2.5 * MALL_BYTES / kv_bytes))
        c0 = qkv.AsymKVCache.empty(w.B, w.Hkv, w.L, w.D, group)
        qkv.quantize_append_kv_asym(kt, vt, c0, 0)
        caches = [c0] + [qkv.AsymKVCache(*(t.clone() for t in c0.tensors()), group) for _ in range(n_copies - 1)]

        def run(i):
            qkv.decode_asym(q, caches[i], w.L, softmax_scale=w.softmax_scale, out=out, workspace=ws)

        for i in range(5):
            run(i % n_copies)
        torch.cuda.synchronize()
        ms = region_ms(torch, run, steps, n_copies)
        alg = kv_bytes + w.B * w.Hq * w.Sq * w.D * 6
        r = {"ms": ms, "kv_bytes": kv_bytes, "GBps": alg / (ms * 1e-3) / 1e9,
             "frac_hbm": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        if int4_ms:
            r["time_vs_int4"] = ms / int4_ms
        res[f"group{group}"] = r
        del caches, c0
        torch.cuda.empty_cache()
    return res


def bench_prefill(torch, qkv, w, iters, bits=4, group=0):
    """Prefill over a cache of ``bits``-bit rows (4: the int4 path), or of
    asymmetric group-wise int4 rows with groups of ``group`` elements."""
    from qkv_inputs import make_qkv
    q_bits, k, v = make_qkv(w)
    if group:
        cache = qkv.AsymKVCache.empty(w.B, w.Hkv, w.L, w.D, group)
        qkv.quantize_append_kv_asym(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), cache, 0)
    elif bits == 4:
        cache = upload_cache(torch, qkv, k, v, 1)[0]
    else:
        cache = qkv.KVCache.empty(w.B, w.Hkv, w.L, w.D, bits=bits)
        qkv.quantize_append_kv(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), cache, 0, bits=bits)
    del k, v
    q = torch.from_numpy(q_bits.view("int16")).cuda().view(torch.bfloat16)
    out = torch.empty((w.B, w.Hq, w.Sq, w.D), dtype=torch.float32, device="cuda")

    def run(_):
        if group:
            qkv.prefill_asym(q, cache, w.L, w.causal, softmax_scale=w.softmax_scale, out=out)
        else:
            qkv.prefill(q, cache, w.L, w.causal, softmax_scale=w.softmax_scale, out=out, bits=bits)

    for i in range(2):
        run(i)
    # back-to-back launches behind a GPU hold (no per-launch event packets,
    # which add ~2 us to a 30 us kernel); the per-launch median beside it
    avg_ms = region_ms(torch, run, iters, 1)
    _, med_ms = per_launch_ms(torch, run, iters, 1)
    fl = prefill_flops(w)
    nbytes = prefill_bytes(w, bits, group)
    res = {"workload": w.name, "bits": bits, "group": group or None, "avg_ms": avg_ms, "median_ms": med_ms,
           "flops": fl,
           "TFLOPs": fl / (avg_ms * 1e-3) / 1e12, "algorithmic_bytes": nbytes,
           "GBps": nbytes / (avg_ms * 1e-3) / 1e9}
    res["frac_mfma"] = res["TFLOPs"] / MFMA_F16_PEAK_TFLOPS
    res["frac_hbm"] = res["GBps"] / HBM_PEAK_GBS
    # the roof that binds: the larger of the two fractions' time floors
    res["bound"] = "hbm" if nbytes / HBM_PEAK_GBS / 1e9 > fl / MFMA_F16_PEAK_TFLOPS / 1e12 else "mfma"
    del cache, q, out
    torch.cuda.empty_cache()
    return res


def bench_hbm_context(torch, iters=10):
    """Achievable-HBM context (not the headline's peak, which stays nominal):
    the library's streaming-read kernel over 1 GiB (qkvb_stream_read, non-temporal loads,
    16-byte loads, four in flight per thread; best of a few grid sizes) and
    torch's 512 MiB device-to-device copy, back to back with events around
    the batch."""
    import ctypes
    blib = ctypes.CDLL(os.path.join(ROOT, "quantized_kv_flashattention_amd", "libqkvfa_bench.so"))
    blib.qkvb_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]
    n = (1 << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty(n // 2, dtype=torch.float32, device="cuda")
    red = torch.empty(65536, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def read(grid):
        def fn():
            if blib.qkvb_stream_read(x.data_ptr(), 1 << 30, red.data_ptr(), grid, stream) != 0:
                raise RuntimeError("qkvb_stream_read failed")
        return fn

    res = {}
    legs = [(f"stream_read_1GiB_grid{g}", read(g), 1 << 30) for g in (1024, 2048, 4096, 8192)]
    legs.append(("copy_512MiB", lambda: y.copy_(x[: n // 2]), 2 * (1 << 29)))
    for name, fn, nbytes in legs:
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        res[name] = {"ms": ms, "GBps": nbytes / (ms * 1e-3) / 1e9, "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    best = max((k for k in res if k.startswith("stream_read")), key=lambda k: res[k]["GBps"])
    res["stream_read_best"] = dict(res[best], leg=best)
    del x, y, red
    torch.cuda.empty_cache()
    return res


def bench_quantize(torch, qkv, w, iters):
    from qkv_inputs import make_qkv
    _, k, _ = make_qkv(w)
    B, H, L, D = k.shape
    kt = torch.from_numpy(k).cuda()
    del k
    codes = torch.empty((B, H, L, D // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((B, H, L), dtype=torch.float16, device="cuda")

    def run(_):
        qkv.quantize_append(kt, codes, scales, 0)

    run(0)
    avg_ms, med_ms = per_launch_ms(torch, run, iters, 1)
    rows = B * H * L
    nbytes = rows * (4 * D + D // 2 + 2)
    del kt, codes, scales
    torch.cuda.empty_cache()
    return {"workload": w.name + ":K", "rows": rows, "avg_ms": avg_ms, "bytes": nbytes,
            "GBps": nbytes / (avg_ms * 1e-3) / 1e9}


def cpu_info():
    """(cores in this process's affinity mask, BLAS pool threads or None, CPU model)."""
    aff = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = None
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return aff, blas, model


def cpu_prefill_sample(w, budget_s, seed=0):
    """The CPU oracle on a bounded sample of a prefill workload: whole (batch,
    head) pairs of a short non-causal workload, or evenly spaced query rows of
    one KV group's heads of a long causal one.  Rate in TFLOP/s of the sampled
    attention (4 D flops per query-key pair) and, for the short workload, GB/s
    of the packed KV bytes the sample's heads read.
    """
    import oracle
    from qkv_inputs import make_qkv
    q_bits, k, v = make_qkv(w, seed)
    G = w.G
    row = w.D // 2 + 2
    t_total, flops, nbytes, done = 0.0, 0.0, 0, 0
    if not w.causal:
        pairs = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
        for b, g in pairs:
            t0 = time.perf_counter()
            kc, ksc = oracle.quantize_rows(k[b:b + 1, g:g + 1])
            vc, vsc = oracle.quantize_rows(v[b:b + 1, g:g + 1])
            oracle.attention(q_bits[b:b + 1, g * G:(g + 1) * G], kc, ksc, vc, vsc, w.L, w.softmax_scale)
            t_total += time.perf_counter() - t0
            done += 1
            flops += 4.0 * w.D * w.Sq * w.L * G
            nbytes += 2 * w.L * row
            if t_total >= budget_s:
                break
        sample = f"{done} of {len(pairs)} (batch, KV head) groups of {w.name} ({G} heads x {w.Sq} rows each)"
    else:
        t0 = time.perf_counter()
        kc, ksc = oracle.quantize_rows(k[:1, :1])
        vc, vsc = oracle.quantize_rows(v[:1, :1])
        t_total += time.perf_counter() - t0
        nbytes = 2 * w.L * row
        off = w.L - w.Sq
        n_rows = 8
        while True:
            rows = sorted({int(r) for r in np.linspace(0, w.Sq - 1, n_rows)})
            t0 = time.perf_counter()
            oracle.attention(q_bits[:1, :G], kc, ksc, vc, vsc, w.L, w.softmax_scale, causal=True,
                             heads=[(0, h) for h in range(G)], rows=rows)
            t_total += time.perf_counter() - t0
            done += len(rows)
            flops += 4.0 * w.D * G * sum(r + off + 1 for r in rows)
            if t_total >= budget_s or n_rows >= w.Sq:
                break
            n_rows *= 2
        sample = (f"{done} query rows (evenly spaced, causal) x {G} heads of KV group (0, 0) of {w.name}, "
                  f"quantizing that group's {w.L} K/V rows once")
    return {"TFLOPs": flops / t_total / 1e12,
            "GBps_packed_kv": None if w.causal else nbytes / t_total / 1e9,
            "seconds": round(t_total, 2), "sample": sample}


def cpu_baseline(w, budget_s):
    """The CPU oracle on a bounded sample of the decode workload (whole KV groups)."""
    import oracle
    from qkv_inputs import make_qkv
    aff, blas, model = cpu_info()
    threads = min(aff, blas) if blas else aff   # the BLAS pool runs within the affinity mask
    q_bits, k, v = make_qkv(w)
    groups = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    done, t_total, nbytes = 0, 0.0, 0
    G = w.G
    for (b, g) in groups:
        ks = k[b:b + 1, g:g + 1]
        vs = v[b:b + 1, g:g + 1]
        t0 = time.perf_counter()
        kc, ksc = oracle.quantize_rows(ks)
        vc, vsc = oracle.quantize_rows(vs)
        oracle.attention(q_bits[b:b + 1, g * G:(g + 1) * G], kc, ksc, vc, vsc, w.L, w.softmax_scale)
        t_total += time.perf_counter() - t0
        done += 1
        nbytes += 2 * w.L * (w.D // 2 + 2)
        if t_total >= budget_s:
            break
    return {
        "value": nbytes / t_total / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"{done} of {len(groups)} (batch, KV head) groups of {w.name} "
                   f"(quantize K/V rows + fp64 attention of {G} heads x {w.L} tokens each), "
                   f"{t_total:.1f} s; GB/s counts packed KV bytes as on the GPU"),
        "affinity_cores": aff, "blas_threads": blas, "cpu_model": model,
    }


def profile_target(target: str, iters: int):
    """Run one kernel `iters` times (for rocprofv3 counter passes) and exit."""
    import torch
    import quantized_kv_flashattention_amd as qkv
    from qkv_inputs import make_qkv, workload
    torch.cuda.set_device(0)
    if target == "copy":
        # plain device copy of known size: calibrates FETCH_SIZE / WRITE_SIZE
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(iters):
            dst.copy_(src)
        torch.cuda.synchronize()
        return
    if target == "paged":
        w = workload("ragged_paged_decode")
        lens, table, _, pool = build_paged(torch, qkv, w)
        q_bits, k1, v1 = make_qkv(w.scaled(L=1))
        q = torch.from_numpy(q_bits.view("int16")).cuda().view(torch.bfloat16)
        k_new, v_new = torch.from_numpy(k1).cuda(), torch.from_numpy(v1).cuda()
        bt, cached = torch.from_numpy(table).cuda(), torch.from_numpy(lens - 1).cuda()
        out = torch.empty((w.B, w.Hq, w.Sq, w.D), dtype=torch.float32, device="cuda")
        for _ in range(iters):
            qkv.decode_paged(q, pool, cached, bt, k_new, v_new, max_kv_len=int(lens.max()),
                             softmax_scale=w.softmax_scale, out=out)
        torch.cuda.synchronize()
        return
    if target == "lowbit":
        # decode only over 4-, 3- and 2-bit caches of the Llama-3-8B shape
        # (one kernel instantiation per width)
        w = workload("llama3_8b_decode")
        q_bits, k, v = make_qkv(w)
        q = torch.from_numpy(q_bits.view("int16")).cuda().view(torch.bfloat16)
        out = torch.empty((w.B, w.Hq, w.Sq, w.D), dtype=torch.float32, device="cuda")
        kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
        del k, v
        for bits in (4, 3, 2):
            c = qkv.KVCache.empty(w.B, w.Hkv, w.L, w.D, bits=bits)
            qkv.quantize_append_kv(kt, vt, c, 0, bits=bits)
            for _ in range(iters):
                qkv.decode(q, c, w.L, softmax_scale=w.softmax_scale, out=out, bits=bits)
            torch.cuda.synchronize()
            del c
        return
    if target == "vit":
        w = workload("vit_b_selfattn")
        q_bits, k, v = make_qkv(w)
        cache = upload_cache(torch, qkv, k, v, 1)[0]
        q = torch.from_numpy(q_bits.view("int16")).cuda().view(torch.bfloat16)
        out = torch.empty((w.B, w.Hq, w.Sq, w.D), dtype=torch.float32, device="cuda")
        for _ in range(iters):
            qkv.prefill(q, cache, w.L, False, softmax_scale=w.softmax_scale, out=out)
        torch.cuda.synchronize()
        return
    if target == "prefill":
        w = workload("causal_prefill_16k")
        q_bits, k, v = make_qkv(w)
        cache = upload_cache(torch, qkv, k, v, 1)[0]
        del k, v
        q = torch.from_numpy(q_bits.view("int16")).cuda().view(torch.bfloat16)
        out = torch.empty((w.B, w.Hq, w.Sq, w.D), dtype=torch.float32, device="cuda")
        for _ in range(max(iters // 4, 3)):
            qkv.prefill(q, cache, w.L, True, softmax_scale=w.softmax_scale, out=out)
        torch.cuda.synchronize()
        return
    w = workload({"decode": "llama3_8b_decode", "long": "long_context_decode"}[target])
    q_bits, k, v = make_qkv(w)
    caches = upload_cache(torch, qkv, k, v, max(4, math.ceil(2.5 * MALL_BYTES / decode_bytes(w)[0])))
    q = torch.from_numpy(q_bits.view("int16")).cuda().view(torch.bfloat16)
    out = torch.empty((w.B, w.Hq, w.Sq, w.D), dtype=torch.float32, device="cuda")
    k_new = torch.from_numpy(k[:, :, -1:].copy()).cuda()
    v_new = torch.from_numpy(v[:, :, -1:].copy()).cuda()
    for i in range(iters):   # the benchmark's step: append the new token + decode, one launch
        qkv.decode_append(q, k_new, v_new, caches[i % len(caches)], w.L - 1, softmax_scale=w.softmax_scale,
                          out=out)
    torch.cuda.synchronize()


COPY_BYTES = 1 << 30


def _counter_per_dispatch(path_dir: str, counter: str, name_re: str):
    """Average value of `counter` per dispatch of kernels matching name_re (KiB)."""
    import csv
    import glob
    import re
    files = glob.glob(os.path.join(path_dir, "**", "*counter_collection.csv"), recursive=True)
    per = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter or not re.search(name_re, r["Kernel_Name"]):
                    continue
                per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    vals = [per[k] for k in sorted(per, key=int)]
    if len(vals) > 4:
        vals = vals[2:]          # skip first dispatches (cold caches, page mapping)
    return (sum(vals) / len(vals)) if vals else None, len(vals)


def summarize_profiles(root: str):
    """Turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes into HBM bytes per
    decode launch.  Expects <root>/{fetch,write}_{decode,copy}/ outputs."""
    fc, nfc = _counter_per_dispatch(os.path.join(root, "fetch_copy"), "FETCH_SIZE", "copyBuffer|copy")
    wc, nwc = _counter_per_dispatch(os.path.join(root, "write_copy"), "WRITE_SIZE", "copyBuffer|copy")
    fd, nfd = _counter_per_dispatch(os.path.join(root, "fetch_decode"), "FETCH_SIZE", "decode_kernel")
    wd, nwd = _counter_per_dispatch(os.path.join(root, "write_decode"), "WRITE_SIZE", "decode_kernel")
    if None in (fc, wc, fd, wd):
        raise SystemExit(f"missing counter data: {fc} {wc} {fd} {wd}")
    f_scale = fc * 1024 / COPY_BYTES     # counter bytes per true byte, reads
    w_scale = wc * 1024 / COPY_BYTES     # same, writes
    from qkv_inputs import workload
    w = workload("llama3_8b_decode")
    alg = decode_bytes(w)[1] + 2 * w.B * w.Hkv * w.D * 4   # + the appended rows (fp32 K and V)
    read_b = fd * 1024 / f_scale
    write_b = wd * 1024 / w_scale
    result = {
        "source_hash": kernel_source_hash(),
        "copy_calibration": {"bytes_copied": COPY_BYTES, "fetch_kib": fc, "write_kib": wc,
                             "fetch_scale": f_scale, "write_scale": w_scale, "dispatches": [nfc, nwc]},
        "kernels": {"decode_llama3_8b": {
            "fetch_kib_raw": fd, "write_kib_raw": wd, "dispatches": [nfd, nwd],
            "read_bytes": read_b, "write_bytes": write_b,
            "bytes_per_launch": read_b + write_b, "algorithmic_bytes": alg,
            "traffic_over_algorithmic": (read_b + write_b) / alg}},
    }
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(result, f, indent=1)
    print(json.dumps(result, indent=1))


def phase_table(torch, qkv, w, launches=10):
    """Per-workgroup phase timestamps of one decode step launch (append 1
    token + decode), from the measurement build libqkvfa_trace.so (the same
    kernels plus s_memrealtime stores).  The step is launched `launches`
    times back to back behind a GPU hold over rotated cache copies; the
    timestamps of the last launch are read back.  Returns the table rows
    (phase, min / median / max over workgroups in microseconds from the
    launch's first workgroup entry) and per-phase durations."""
    import ctypes
    path = os.path.join(ROOT, "quantized_kv_flashattention_amd", "libqkvfa_trace.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: build it with `python quantized_kv_flashattention_amd/build.py`")
    qkv._LIB_PATH = path
    qkv._lib = qkv._load()
    qkv._lib.qkv_trace_read.restype = ctypes.c_int
    qkv._lib.qkv_trace_read.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    from qkv_inputs import make_qkv
    q_bits, k, v = make_qkv(w)
    kv_bytes, _ = decode_bytes(w)
    n_copies = max(4, math.ceil(2.5 * MALL_BYTES / kv_bytes))
    caches = upload_cache(torch, qkv, k, v, n_copies)
    k_new = torch.from_numpy(k[:, :, -1:].copy()).cuda()
    v_new = torch.from_numpy(v[:, :, -1:].copy()).cuda()
    del k, v
    q = torch.from_numpy(q_bits.view("int16")).cuda().view(torch.bfloat16)
    out = torch.empty((w.B, w.Hq, w.Sq, w.D), dtype=torch.float32, device="cuda")
    ns = qkv.decode_auto_splits(w.B, w.Hq, w.Hkv, w.Sq, w.L, w.D)
    ws = torch.zeros(max(qkv.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.L, w.D), 1), dtype=torch.uint8,
                     device="cuda")

    def step(i):
        qkv.decode_append(q, k_new, v_new, caches[i % n_copies], w.L - 1, softmax_scale=w.softmax_scale, out=out,
                          workspace=ws)

    for i in range(5):
        step(i)
    torch.cuda.synchronize()
    avg_ms = region_ms(torch, step, launches, n_copies)
    n_wg = ns * w.B * w.Hkv
    buf = np.zeros((n_wg, 16), dtype=np.uint64)
    rc = qkv._lib.qkv_trace_read(buf.ctypes.data, n_wg)
    if rc != 0:
        raise RuntimeError(f"qkv_trace_read failed ({rc})")
    t = buf.astype(np.float64) / 100.0          # s_memrealtime: 100 MHz -> microseconds
    t0 = t[:, 0].min()
    merged = buf[:, 13] == 1
    loop_end = t[:, 2:10].max(axis=1)
    cols = {"entry": t[:, 0], "chunk loop start": t[:, 1], "first wave done": t[:, 2:10].min(axis=1),
            "last wave done": loop_end, "wave merge + partial written": t[:, 10],
            "ticket drawn": t[:, 11], "exit (non-merging)": t[:, 12][~merged],
            "exit (merging)": t[:, 12][merged]}
    rows = []
    for name, x in cols.items():
        x = x - t0
        rows.append({"phase": name, "n": int(x.size), "min_us": round(float(x.min()), 2),
                     "median_us": round(float(np.median(x)), 2), "max_us": round(float(x.max()), 2)})
    dur = {
        "launch (first entry to last exit)": float(t[:, 12].max() - t0),
        "loop, per workgroup (start to last wave)": float(np.median(loop_end - t[:, 1])),
        "wave spread inside a workgroup (last - first wave done)": float(np.median(loop_end - t[:, 2:10].min(axis=1))),
        "wave merge + partial (last wave done to written)": float(np.median(t[:, 10] - loop_end)),
        "store wait + ticket (written to ticket)": float(np.median(t[:, 11] - t[:, 10])),
        "split merge (ticket to exit, merging workgroups)": float(np.median((t[:, 12] - t[:, 11])[merged])),
        "last loop end to last exit": float(t[:, 12].max() - loop_end.max()),
    }
    res = {"workload": w.name, "n_split": ns, "workgroups": n_wg, "launches": launches,
           "avg_launch_ms_trace_build": avg_ms, "rows": rows,
           "durations_us": {k: round(v, 2) for k, v in dur.items()}}
    qkv._LIB_PATH = os.path.join(ROOT, "quantized_kv_flashattention_amd", "libqkvfa.so")
    qkv._lib = qkv._load()
    return res


def print_phase_table(res):
    print(f"workload {res['workload']}: {res['workgroups']} workgroups ({res['n_split']} splits), "
          f"last of {res['launches']} back-to-back launches; trace build {res['avg_launch_ms_trace_build'] * 1e3:.2f} "
          f"us per launch")
    print()
    print("| phase (us from the first workgroup's entry) | workgroups | min | median | max |")
    print("|---|---|---|---|---|")
    for r in res["rows"]:
        print(f"| {r['phase']} | {r['n']} | {r['min_us']:.2f} | {r['median_us']:.2f} | {r['max_us']:.2f} |")
    print()
    print("| duration | us |")
    print("|---|---|")
    for k, v in res["durations_us"].items():
        print(f"| {k} | {v:.2f} |")
    print()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", choices=["all", "headline", "decode", "prefill"], default="all")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--profile-target", choices=["decode", "long", "paged", "prefill", "vit", "copy", "lowbit"],
                    default=None,
                    help="run one kernel repeatedly for rocprofv3 counter passes, print nothing")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="write profiles/traffic.json from rocprofv3 FETCH_SIZE/WRITE_SIZE passes in DIR")
    ap.add_argument("--phase-table", action="store_true",
                    help="print per-workgroup phase timestamps of the Llama-3-8B and 128K decode steps "
                         "(measurement build libqkvfa_trace.so) as markdown tables, then a JSON line")
    args = ap.parse_args()
    if args.phase_table:
        import torch
        import quantized_kv_flashattention_amd as qkv
        from qkv_inputs import workload
        torch.cuda.set_device(0)
        res = [phase_table(torch, qkv, workload(n)) for n in ("llama3_8b_decode", "long_context_decode")]
        for r in res:
            print_phase_table(r)
        print(json.dumps(res), flush=True)
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.profile_target:
        profile_target(args.profile_target, 20)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_kv_flashattention_amd as qkv
    from qkv_inputs import workload
    torch.cuda.set_device(0)
    dev = torch.cuda.get_device_properties(0)
    log(f"device: {dev.name} CUs={dev.multi_processor_count}")

    w3 = workload("llama3_8b_decode")
    head = bench_decode(torch, qkv, w3, args.steps, args.warmup, with_append=True)
    log("headline:", json.dumps(head))
    secondary = {}
    if args.only in ("all", "decode"):
        secondary["long_context_decode"] = bench_decode(torch, qkv, workload("long_context_decode"),
                                                        max(args.steps // 2, 10), 5, with_append=True)
        log("long:", json.dumps(secondary["long_context_decode"]))
        secondary["ragged_paged_decode"] = bench_paged(torch, qkv, workload("ragged_paged_decode"),
                                                       max(args.steps // 2, 10))
        log("paged:", json.dumps(secondary["ragged_paged_decode"]))
        secondary["int8_buffer_decode"] = bench_buffered(torch, qkv, w3, max(args.steps, 20))
        log("buffered:", json.dumps(secondary["int8_buffer_decode"]))
        secondary["lowbit_decode"] = bench_lowbit(torch, qkv, w3, max(args.steps, 20))
        log("lowbit:", json.dumps(secondary["lowbit_decode"]))
        secondary["asym_group_decode"] = bench_asym(torch, qkv, w3, max(args.steps, 20),
                                                    secondary["lowbit_decode"]["4bit"]["ms"])
        log("asym:", json.dumps(secondary["asym_group_decode"]))
    if args.only in ("all", "prefill"):
        secondary["causal_prefill_16k"] = bench_prefill(torch, qkv, workload("causal_prefill_16k"), 10)
        log("prefill:", json.dumps(secondary["causal_prefill_16k"]))
        secondary["vit_b_selfattn"] = bench_prefill(torch, qkv, workload("vit_b_selfattn"), 20)
        log("vit:", json.dumps(secondary["vit_b_selfattn"]))
        secondary["causal_prefill_16k_lowbit"] = {
            f"{b}bit": bench_prefill(torch, qkv, workload("causal_prefill_16k"), 6, bits=b) for b in (2, 3)}
        log("prefill lowbit:", json.dumps(secondary["causal_prefill_16k_lowbit"]))
        secondary["causal_prefill_16k_asym"] = {
            f"group{g}": bench_prefill(torch, qkv, workload("causal_prefill_16k"), 6, group=g) for g in (128, 64, 32)}
        log("prefill asym:", json.dumps(secondary["causal_prefill_16k_asym"]))
    if args.only == "all":
        secondary["hbm_context"] = bench_hbm_context(torch)
        log("hbm context:", json.dumps(secondary["hbm_context"]))
        secondary["quantize_append"] = bench_quantize(torch, qkv, w3, 20)
        log("quantize:", json.dumps(secondary["quantize_append"]))

    cpu = cpu_baseline(w3, args.cpu_budget)
    if args.only == "all":
        cpu["other_configs"] = {n: cpu_prefill_sample(workload(n), args.cpu_budget / 2)
                                for n in ("vit_b_selfattn", "causal_prefill_16k")}
    log("cpu:", json.dumps(cpu))

    value = head["step_GBps_packed_kv"]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w3.name, "B": w3.B, "Hq": w3.Hq, "Hkv": w3.Hkv, "D": w3.D,
                   "Sq": w3.Sq, "kv_len": w3.L, "kv_format": "int4 + fp16 scale per (token, KV head)",
                   "step": "append 1 token (K,V) + split-K decode, one launch", "n_split": head["n_split"],
                   "cache_copies_rotated": head["cache_copies"]},
        "roofline": {
            "bound": "hbm",
            "achieved": round(head["kernel_GBps"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head["kernel_frac_hbm"], 4),
            "traffic": measured_traffic("decode_llama3_8b"),
        },
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Seeded synthetic inputs for int4-KV attention: workload shapes and raw tensors.

This module is shared by the CPU oracle (``oracle/``), the tests and the
benchmark.  It holds no arithmetic of the attention method: it only draws
random numbers and rounds the query to bfloat16 (the storage type the
library's query operand has).  Quantization of K/V is *not* done here; each
side (oracle, GPU library) quantizes the fp32 K/V it receives on its own.

Workload shapes stand in for the pages' real workloads, whose datasets and
model weights are not available:

* tiny decode (parity case),
* ViT-B/DeiT shaped self-attention (QFlash abstract, "Attention Quantization"
  topic listing: ViT/DeiT/Swin workloads),
* Llama-3-8B shaped GQA decode with 8 KV heads (TurboAttention, arXiv
  2412.08585 §5 ablation on "8-head configuration per key/value cache"),
  with channel-wise outliers (same paper §3.1: outliers concentrate in a few
  channels of K/V),
* long-context decode at 128K tokens (Open-TQ-Metal abstract: Llama 3.1 70B at
  128K context with an int4 KV cache),
* causal GQA prefill at 16K tokens (TurboAttention §5: 4k-32k contexts),
* a ragged serving batch: 64 Llama-3-8B shaped sequences of mixed lengths in
  a shared page pool (TurboAttention §2.1: every decode step appends each
  sequence's new token and attends its cache; §5 serves batches of up to 64).

Distributions: every raw value is N(0, 1) in fp32 from numpy's PCG64, seeded
by ``SeedSequence([seed, config_index])`` and spawned into independent streams
for Q, K, V and the outlier-channel choice.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_inputs",
    "make_qkv",
    "ragged_layout",
    "pool_rows",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and structure of one synthetic attention workload."""

    index: int          # position in the workload table (also the seed stream)
    name: str
    mode: str           # "decode" or "prefill"
    B: int              # batch
    Hq: int             # query heads
    Hkv: int            # KV heads (Hq % Hkv == 0; G = Hq // Hkv)
    D: int              # head dim
    Sq: int             # query rows per (batch, head)
    L: int              # cached KV tokens
    causal: bool
    outlier_frac: float = 0.0    # fraction of Hkv*D channels scaled x outlier_gain
    outlier_gain: float = 8.0
    len_min: int = 0    # ragged batch: lengths uniform in [len_min, L] (0: every sequence has L)
    page_size: int = 0  # paged cache: rows per page (0: contiguous cache)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def softmax_scale(self) -> float:
        """fp32 value of 1/sqrt(D), as a Python float."""
        return float(np.float32(1.0 / math.sqrt(self.D)))

    def scaled(self, **kw) -> "Workload":
        """Same structure with some sizes replaced (for small parity cases)."""
        return dataclasses.replace(self, **kw)


WORKLOADS = [
    Workload(0, "tiny_decode", "decode", B=1, Hq=2, Hkv=2, D=64, Sq=1, L=256, causal=False),
    Workload(1, "vit_b_selfattn", "prefill", B=64, Hq=12, Hkv=12, D=64, Sq=197, L=197, causal=False),
    Workload(2, "llama3_8b_decode", "decode", B=16, Hq=32, Hkv=8, D=128, Sq=1, L=8192, causal=False,
             outlier_frac=0.01),
    Workload(3, "long_context_decode", "decode", B=1, Hq=64, Hkv=8, D=128, Sq=1, L=131072, causal=False),
    Workload(4, "causal_prefill_16k", "prefill", B=1, Hq=32, Hkv=8, D=128, Sq=16384, L=16384, causal=True),
    Workload(5, "ragged_paged_decode", "decode", B=64, Hq=32, Hkv=8, D=128, Sq=1, L=16384, causal=False,
             len_min=512, page_size=64),
]


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for w in WORKLOADS:
        if w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bfloat16 (round-to-nearest-even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(index: int, seed: int):
    ss = np.random.SeedSequence([seed, index])
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(4)]


def make_qkv(w: Workload, seed: int = 0):
    """Raw inputs of workload ``w``.

    Returns ``(q_bits, k, v)``: ``q_bits`` uint16 bf16 bits ``[B, Hq, Sq, D]``;
    ``k``, ``v`` fp32 ``[B, Hkv, L, D]`` (outlier channels already scaled).
    """
    rq, rk, rv, ro = _streams(w.index, seed)
    q = rq.standard_normal((w.B, w.Hq, w.Sq, w.D), dtype=np.float32)
    q_bits = f32_to_bf16_bits(q)
    del q
    k = rk.standard_normal((w.B, w.Hkv, w.L, w.D), dtype=np.float32)
    v = rv.standard_normal((w.B, w.Hkv, w.L, w.D), dtype=np.float32)
    if w.outlier_frac > 0:
        n_ch = w.Hkv * w.D
        n_out = max(1, int(round(w.outlier_frac * n_ch)))
        gain = np.float32(w.outlier_gain)
        for t in (k, v):
            ch = ro.choice(n_ch, size=n_out, replace=False)
            for c in ch:
                h, d = divmod(int(c), w.D)
                t[:, h, :, d] *= gain   # exact: power-of-two gain
    return q_bits, k, v


def make_inputs(w: Workload, seed: int = 0):
    """Dict form of :func:`make_qkv` with the workload attached."""
    q_bits, k, v = make_qkv(w, seed)
    return {"workload": w, "q_bits": q_bits, "k": k, "v": v}


def ragged_layout(w: Workload, seed: int = 0):
    """Lengths and page table of a ragged, paged workload.

    Returns ``(lens, table, num_pages)``: ``lens`` int32 ``[B]`` attended rows
    per sequence, uniform in ``[len_min, L]``; ``table`` int32 ``[B,
    ceil(L / page_size)]``, the pages of every sequence drawn without
    replacement from a shuffled pool of exactly the pages needed (entries past
    a sequence's last page are -1); ``num_pages`` the pool size.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, w.index, 7])))
    lo = w.len_min if w.len_min > 0 else w.L
    lens = rng.integers(lo, w.L + 1, size=w.B).astype(np.int32)
    P = w.page_size
    used = [-(-int(L) // P) for L in lens]
    num_pages = int(sum(used))
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((w.B, -(-w.L // P)), -1, np.int32)
    k = 0
    for b, u in enumerate(used):
        table[b, :u] = perm[k:k + u]
        k += u
    return lens, table, num_pages


def pool_rows(w: Workload, num_pages: int, chunk_pages: int, seed: int = 0):
    """fp32 N(0, 1) K and V rows of a page pool, ``chunk_pages`` pages at a time.

    Yields ``(first_page, k, v)`` with ``k``, ``v`` fp32 ``[n, Hkv, page_size, D]``.
    """
    ss = np.random.SeedSequence([seed, w.index, 11])
    rk, rv = (np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(2))
    for p0 in range(0, num_pages, chunk_pages):
        n = min(chunk_pages, num_pages - p0)
        shape = (n, w.Hkv, w.page_size, w.D)
        yield p0, rk.standard_normal(shape, dtype=np.float32), rv.standard_normal(shape, dtype=np.float32)

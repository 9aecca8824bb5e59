"""CPU oracle for int4-KV attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The product path (the HIP library and its Python
binding) never imports, links or runs anything from here, and this package
imports nothing from the product path.  The two share only the seeded input
generator (``qkv_inputs``), which holds none of the method's arithmetic.

What the oracle computes is the plain definition of the method's result,
written out (the fused, tiled, online-softmax kernels reach the same value in
exact arithmetic):

* ``quantize``: per-row int4 quantization with one fp16 scale per (token, KV
  head), in fp32 as the quantizer is specified (scale = fp16(absmax / 7) with
  IEEE fp32 division then round-to-nearest-even to fp16; code =
  clamp(rint(x / float(scale)), -8, 7); a zero scale gives all-zero codes),
  two's-complement nibbles packed low-nibble-first;
* ``attention``: dequantize K/V exactly to fp64, then plain fp64
  softmax(Q K^T * scale) V with an optional bottom-right causal mask, plus the
  natural-log log-sum-exp of each row;
* ``attention_partial`` / ``lse_merge``: the same attention restricted to a
  key range, and the log-sum-exp merge of such partial results (the
  definition the split-K decode reaches);
* ``lowbit``: 2- and 3-bit rows (the int4 rule widened to b bits, packing
  of 2-bit rows and of 3-bit rows as two bit planes) and attention over them;
* ``buffer``: the INT8 decode buffer -- universal scale from the cache's
  value range, symmetric clamped 8-bit codes, the flush to int4, and
  attention over int4 rows followed by buffered INT8 rows;
* ``asym``: asymmetric group-wise int4 rows (a scale and a zero point per
  group of consecutive elements) and attention over them.

Every function is pinned by tests in ``tests/test_oracle_*.py`` against hand
derived examples, exact rational arithmetic, brute force on tiny inputs,
closed forms and invariants.
"""
from .quantize import quantize_rows, dequantize_rows, quantize_append, dequantize_cache
from .attention import attention, attention_partial, lse_merge
from .buffer import buffer_scale, quantize_int8, dequantize_int8, flush_rows, attention_buffered
from .lowbit import (row_bytes, quantize_rows_bits, unpack_bits, dequantize_rows_bits, dequantize_cache_bits,
                     attention_bits)
from .asym import (quantize_rows_asym, unpack_asym, dequantize_rows_asym, dequantize_cache_asym, attention_asym,
                   cache_order, to_cache_order, from_cache_order)

__all__ = [
    "quantize_rows",
    "dequantize_rows",
    "quantize_append",
    "dequantize_cache",
    "attention",
    "attention_partial",
    "lse_merge",
    "buffer_scale",
    "quantize_int8",
    "dequantize_int8",
    "flush_rows",
    "attention_buffered",
    "row_bytes",
    "quantize_rows_bits",
    "unpack_bits",
    "dequantize_rows_bits",
    "dequantize_cache_bits",
    "attention_bits",
    "quantize_rows_asym",
    "unpack_asym",
    "dequantize_rows_asym",
    "dequantize_cache_asym",
    "attention_asym",
    "cache_order",
    "to_cache_order",
    "from_cache_order",
]

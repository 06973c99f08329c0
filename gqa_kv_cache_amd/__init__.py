"""Grouped-query attention over a KV cache on AMD Instinct MI355X (gfx950).

The computation lives in ``libgqa.so`` (hand-written HIP kernels behind the
C ABI of ``include/gqa.h``); this package is its Python binding.

* ``decode(q, k_cache, v_cache, seqlens)`` -- one new token per sequence.
* ``decode_noalloc(q, k_cache, v_cache, seqlens, out)`` -- the same without
  any allocation (split partials in the library's static device scratch).
* ``decode_ex(q, k_cache, v_cache, seqlens, ...)`` -- several new tokens per
  sequence, append, FP8 (E4M3 or E5M2) cache, paged cache, sliding window.
* ``prefill(q, k, v, causal=True)`` -- the whole prompt at once.
* count helpers: ``kv_cache_elems``, ``decode_bytes``, ``decode_flops``,
  ``prefill_flops``, ``prefill_bytes``.
"""
from ._native import (BF16, EXPORTS, F32, FP8_E4M3, FP8_E5M2, LIBRARY_PATH, GqaError, Status,  # noqa: F401
                      decode, decode_bytes, decode_ex, decode_flops, decode_noalloc, decode_num_splits,
                      decode_workspace_size,
                      kv_cache_elems, load, prefill, prefill_bytes, prefill_flops, status_str)

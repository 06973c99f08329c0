"""Oracle for grouped-query attention over a KV cache -- TEST INFRASTRUCTURE.

A plain, slow, obviously correct CPU implementation used only to check the
GPU library: by the test suite, by the smoke check and by the benchmark's
CPU-baseline leg.  The product path (``gqa_kv_cache_amd``) never imports it,
and it imports nothing from the product path.

* ``reference``: fp64 C implementation (``gqa_oracle.c``) behind ctypes --
  decode, prefill, and separately written MHA and MQA decoders.
* ``brute``: pure-Python fp64 brute force for tiny inputs.
* ``counts``: exact integer KV-cache sizes, traffic and FLOP counts.

Every function is pinned by tests in ``tests/test_oracle_*.py`` against
closed forms, special cases, invariants and the pages' printed numbers.
"""
from . import brute, counts, reference  # noqa: F401

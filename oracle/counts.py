"""Exact integer counts of KV-cache size, traffic and work -- TEST INFRASTRUCTURE.

Written independently of the library's own count functions, from the pages'
formulas:

* KV-cache elements = 2 x layers x KV heads x length x head dim (the leading 2
  is K and V): "查询头保持不变，只减少键值头" (ttlab lesson), section
  "什么减少，什么不减少"; bytes multiply by the element size, and by batch:
  "GQA reading notes" (zhongzhuzhou.org) section 3 (KV 缓存) equation S_KV;
  "从MHA到GQA" (gzher.com) cache formula 2*B*N*L*H_kv*d_h*b; "GQA 深入理解"
  (zulogic.cn) section 3.1.
* Per-step decode traffic: K and V of every cached row are read once per KV
  head, not per query head ("GQA reading notes", Algorithm 2 walkthrough and
  the formal definition T_KV = 2 G L d_k B bytes).  Algorithmic bytes of one
  decode call add the query and the output once each.
* Multiplication counts of one attention layer over n positions (ttlab lesson,
  same section): scores h*n*n*d and weighted sum h*n*n*d -- no group count in
  either; K and V projections n*d_model*(g*d) each.
* A multiply-add is 2 FLOP.  Decode FLOP = 4*Hq*d*sum(seqlens); causal
  prefill counts only the P(P+1)/2 unmasked query-key pairs.
"""
from __future__ import annotations


def kv_cache_elems(length: int, kv_heads: int, head_dim: int, layers: int = 1,
                   batch: int = 1) -> int:
    return 2 * layers * kv_heads * length * head_dim * batch


def kv_cache_bytes(length: int, kv_heads: int, head_dim: int, elt_bytes: int,
                   layers: int = 1, batch: int = 1) -> int:
    return kv_cache_elems(length, kv_heads, head_dim, layers, batch) * elt_bytes


def decode_kv_read_bytes(seqlens, kv_heads: int, head_dim: int, elt_bytes: int) -> int:
    """K and V bytes one decode call must read: every valid row, once per KV head."""
    return sum(2 * int(n) * kv_heads * head_dim * elt_bytes for n in seqlens)


def decode_bytes(seqlens, q_heads: int, kv_heads: int, head_dim: int, elt_bytes: int) -> int:
    """Algorithmic bytes of one decode call: K+V read once, plus Q in and O out."""
    batch = len(seqlens)
    qo = 2 * batch * q_heads * head_dim * elt_bytes
    return decode_kv_read_bytes(seqlens, kv_heads, head_dim, elt_bytes) + qo


def decode_flops(seqlens, q_heads: int, head_dim: int) -> int:
    """2 FLOP per multiply-add, scores plus weighted sum, per query head."""
    return sum(4 * q_heads * head_dim * int(n) for n in seqlens)


def prefill_pairs(prompt: int, causal: bool) -> int:
    return prompt * (prompt + 1) // 2 if causal else prompt * prompt


def prefill_flops(batch: int, prompt: int, q_heads: int, head_dim: int, causal: bool) -> int:
    return 4 * batch * q_heads * head_dim * prefill_pairs(prompt, causal)


def prefill_bytes(batch: int, prompt: int, q_heads: int, kv_heads: int, head_dim: int,
                  elt_bytes: int) -> int:
    """Q in, K and V in, O out, each once."""
    return batch * prompt * head_dim * elt_bytes * (2 * q_heads + 2 * kv_heads)


def attention_mults(q_heads: int, n: int, head_dim: int) -> dict:
    """Multiplications of one attention layer pass over n positions (no group count)."""
    return {"scores": q_heads * n * n * head_dim, "weighted_sum": q_heads * n * n * head_dim}


def kv_projection_mults(n: int, d_model: int, kv_heads: int, head_dim: int) -> dict:
    return {"k_proj": n * d_model * kv_heads * head_dim, "v_proj": n * d_model * kv_heads * head_dim}

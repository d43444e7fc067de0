"""Byte and block accounting (float-free integer formulas).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Pages cited in this file:
  [3] "PagedAttention and vLLM: Virtual Memory for the KV Cache" (passgenai.com)
  [4] "What is paged attention?" (netraruntime.com/learn/paged-attention)
"""
from __future__ import annotations


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, seq_len: int,
                   bytes_per_elem: int) -> int:
    """Cache a sequence genuinely needs: K and V (the factor 2) for every
    layer, KV head, head dimension and token ([3], the FAQ answer on whether
    paging shrinks the cache, restating lesson 12-05's formula)."""
    return 2 * layers * kv_heads * head_dim * seq_len * bytes_per_elem


def blocks_for_tokens(t: int, block_size: int = 16) -> int:
    """A sequence of t tokens holds ceil(t / B) blocks ([4], "How it works")."""
    return -(-t // block_size)


def waste_slots(t: int, block_size: int = 16) -> int:
    """Unused slots of the last, partially filled block (0 .. B-1)."""
    return blocks_for_tokens(t, block_size) * block_size - t


def decode_call_bytes(context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                      elem_bytes: int, block_size: int = 16) -> dict:
    """Algorithmic bytes one decode-attention call must move: every live K and
    V element once (exact lengths, no padding to whole blocks), the queries,
    the fp32 outputs, the live block-table entries and the lengths."""
    lens = [int(t) for t in context_lens]
    S = len(lens)
    kv = sum(lens) * num_kv_heads * head_dim * elem_bytes * 2
    q = S * num_q_heads * head_dim * elem_bytes
    out = S * num_q_heads * head_dim * 4
    tables = sum(blocks_for_tokens(t, block_size) for t in lens) * 4
    return {"kv": kv, "q": q, "out": out, "tables": tables, "lens": 4 * S,
            "total": kv + q + out + tables + 4 * S}

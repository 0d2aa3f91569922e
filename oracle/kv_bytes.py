"""KV-cache byte accounting (oracle; test infrastructure).

The KV-size product of the vLLM page ("vLLM — PagedAttention으로 ...", section
"KV Cache가 왜 병목인가"): K and V (factor 2) for every layer, head, head-dim
element and token, times the bytes of one element.

Per decode step each sequence's K and V are read once per kv head -- not once
per q head -- so the algorithmic bytes of one layer's decode are
sum_i L_i * 2 * Hkv * D * elem_bytes (logical), or, when sequences share prefix
blocks, the same product over the distinct (physical block, offset) slots read
(unique).
"""
import numpy as np


def kv_cache_bytes(num_layers, num_kv_heads, head_dim, num_tokens, elem_bytes):
    return 2 * num_layers * num_kv_heads * head_dim * num_tokens * elem_bytes


def decode_kv_bytes_logical(context_lens, num_kv_heads, head_dim, elem_bytes):
    return kv_cache_bytes(1, num_kv_heads, head_dim, int(np.sum(np.asarray(context_lens, dtype=np.int64))), elem_bytes)


def decode_kv_bytes_unique(block_tables, context_lens, block_size, num_kv_heads, head_dim, elem_bytes):
    slots = set()
    for i, L in enumerate(np.asarray(context_lens)):
        for t in range(int(L)):
            slots.add((int(block_tables[i][t // block_size]), t % block_size))
    return kv_cache_bytes(1, num_kv_heads, head_dim, len(slots), elem_bytes)

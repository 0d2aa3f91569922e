"""Where a cached K or V element lives in the physical pool (oracle; test infrastructure).

The pages fix only that the cache is cut into fixed-size blocks that a block
table maps from logical to physical ("vLLM — PagedAttention으로 ...", section
"PagedAttention — OS 가상 메모리에서 영감"); the order of elements inside a block
is this library's choice.  The reading taken here, for N physical blocks, Hkv kv
heads, block size bs (a multiple of 16) and head dim D (a multiple of 8): the
block is the outermost index, then the kv head, then the block's tokens, then
the dims -- K and V alike, so one token's K (or V) for one kv head is one
contiguous row of D values.

Two independent statements of it follow: an element-offset formula (used by the
append and by the brute-force reference) and a reshape view of the whole pool
in logical [N, Hkv, bs, D] order (used by the decode oracle).  The tests check
each against the other.
"""
import numpy as np


def k_offset(n, h, t, d, num_kv_heads, block_size, head_dim):
    """Flat element offset of K[block n, kv head h, token t of the block, dim d]."""
    return ((n * num_kv_heads + h) * block_size + t) * head_dim + d


def v_offset(n, h, t, d, num_kv_heads, block_size, head_dim):
    """Flat element offset of V[block n, kv head h, token t of the block, dim d]."""
    return ((n * num_kv_heads + h) * block_size + t) * head_dim + d


def k_logical(k_flat: np.ndarray, num_blocks, num_kv_heads, block_size, head_dim) -> np.ndarray:
    """View of the K pool as [N, Hkv, bs, D] (no copy)."""
    return k_flat.reshape(num_blocks, num_kv_heads, block_size, head_dim)


def v_logical(v_flat: np.ndarray, num_blocks, num_kv_heads, block_size, head_dim) -> np.ndarray:
    """View of the V pool as [N, Hkv, bs, D] (no copy)."""
    return v_flat.reshape(num_blocks, num_kv_heads, block_size, head_dim)


def check_shape(num_kv_heads, block_size, head_dim):
    if block_size % 16 or block_size <= 0:
        raise ValueError("block_size must be a positive multiple of 16")
    if head_dim % 8 or head_dim <= 0:
        raise ValueError("head_dim must be a positive multiple of 8")
    if num_kv_heads <= 0:
        raise ValueError("num_kv_heads must be positive")

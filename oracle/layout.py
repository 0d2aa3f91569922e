"""Where a cached K or V element lives in the physical pool (oracle; test infrastructure).

The pages fix only that the cache is cut into fixed-size blocks that a block
table maps from logical to physical ("vLLM — PagedAttention으로 ...", section
"PagedAttention — OS 가상 메모리에서 영감"); the order of elements inside a block
is this library's choice.  The reading taken here, for N physical blocks, Hkv kv
heads, block size bs (a multiple of 16) and head dim D (a multiple of 8):

* a block is the outermost index, then the kv head, then the block's tokens in
  groups of 16 ("sub-tiles");
* K inside a sub-tile: [D/8][16 tokens][8 dims] -- 16-byte runs of 8 dims,
  token-major within each run;
* V inside a sub-tile: [D][16 tokens] -- each dim's 16 token values together.

Two independent statements of it follow: an element-offset formula (used by the
append and by the brute-force reference) and a reshape/transpose view of the
whole pool in logical [N, Hkv, bs, D] order (used by the decode oracle).  The
tests check each against the other.
"""
import numpy as np


def k_offset(n, h, t, d, num_kv_heads, block_size, head_dim):
    """Flat element offset of K[block n, kv head h, token t of the block, dim d]."""
    sub = (n * num_kv_heads + h) * (block_size // 16) + t // 16
    return ((sub * (head_dim // 8) + d // 8) * 16 + t % 16) * 8 + d % 8


def v_offset(n, h, t, d, num_kv_heads, block_size, head_dim):
    """Flat element offset of V[block n, kv head h, token t of the block, dim d]."""
    sub = (n * num_kv_heads + h) * (block_size // 16) + t // 16
    return (sub * head_dim + d) * 16 + t % 16


def k_logical(k_flat: np.ndarray, num_blocks, num_kv_heads, block_size, head_dim) -> np.ndarray:
    """View of the K pool as [N, Hkv, bs, D] (no copy)."""
    a = k_flat.reshape(num_blocks, num_kv_heads, block_size // 16, head_dim // 8, 16, 8)
    # -> [N, Hkv, bs/16, 16, D/8, 8] -> [N, Hkv, bs, D]
    return a.transpose(0, 1, 2, 4, 3, 5).reshape(num_blocks, num_kv_heads, block_size, head_dim)


def v_logical(v_flat: np.ndarray, num_blocks, num_kv_heads, block_size, head_dim) -> np.ndarray:
    """View of the V pool as [N, Hkv, bs, D]."""
    a = v_flat.reshape(num_blocks, num_kv_heads, block_size // 16, head_dim, 16)
    return a.transpose(0, 1, 2, 4, 3).reshape(num_blocks, num_kv_heads, block_size, head_dim)


def check_shape(num_kv_heads, block_size, head_dim):
    if block_size % 16 or block_size <= 0:
        raise ValueError("block_size must be a positive multiple of 16")
    if head_dim % 8 or head_dim <= 0:
        raise ValueError("head_dim must be a positive multiple of 8")
    if num_kv_heads <= 0:
        raise ValueError("num_kv_heads must be positive")

"""Paged prefill attention, from its definition (oracle; test infrastructure).

Prefill takes every token of a prompt in one pass ("vLLM — PagedAttention으로
...", section "Prefill vs Decode": all prompt tokens at once, mostly matrix
products; "Nano-vLLM로 배우는 ...", section "Prefill vs Decode: 추론이 “한 번에
읽고, 한 글자씩 쓴다”").  Each new token attends over the K/V of itself and of
every earlier position, never a later one (the causal mask of "[Hacker News
요약] ... 'Tiny-vLLM' 직접 구축하기", section "고성능 추론을 위한 고급 최적화
기법", with the same attention formula and GQA grouping as decode).  The K/V
live in the paged pool, read through the block table as in decode.

Readings taken where the pages are silent:
* the K/V of all L_i context positions of sequence i, the new ones included,
  are in the pool before the call (the multi-token kv_append runs first);
* the call's n_i new tokens are the last n_i positions of the context, so new
  token j sits at position L_i - n_i + j; the positions before them are a
  prefix already in the pool (a prompt's cached prefix blocks, "Nano-vLLM로
  배우는 ...", section "KV 캐시와 Block Manager", or an earlier chunk);
* the new tokens of all sequences are packed in one array, sequence i's at
  rows query_start[i] .. query_start[i+1] - 1;
* everything else (scale, GQA order, rounding, empty sequences) as in
  oracle.attention.

float64 throughout; one query position at a time, no blocking or online
softmax.
"""
import numpy as np

from .attention import attend, gather_context, kv_head_of
from .layout import check_shape, k_logical, v_logical
from .numerics import bits_to_f64, scale_as_passed


def position_of(context_len: int, num_new: int, j: int) -> int:
    """Context position of new token j of a sequence whose last num_new positions are new."""
    return context_len - num_new + j


def visible_keys(position: int) -> int:
    """Keys a query at this position attends to: positions 0 .. position."""
    return position + 1


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, *, dtype, num_blocks,
            num_kv_heads, block_size):
    """Causal attention of every new token over its sequence's paged context.

    q: uint16 bits [T, Hq, D], T = query_start[B]; k_cache, v_cache: uint16 pools in
    the layout of ``oracle.layout``; block_tables int [B, M]; context_lens int [B];
    query_start int [B + 1], non-decreasing, query_start[0] = 0.  Returns float64
    [T, Hq, D]."""
    q = np.asarray(q)
    T, Hq, D = q.shape
    check_shape(num_kv_heads, block_size, D)
    if Hq % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // num_kv_heads
    qs = np.asarray(query_start, dtype=np.int64)
    B = len(qs) - 1
    assert qs[0] == 0 and qs[-1] == T and np.all(np.diff(qs) >= 0), "bad query_start"
    k_log = k_logical(np.asarray(k_cache), num_blocks, num_kv_heads, block_size, D)
    v_log = v_logical(np.asarray(v_cache), num_blocks, num_kv_heads, block_size, D)
    scale64 = scale_as_passed(scale)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for i in range(B):
        s0, s1 = int(qs[i]), int(qs[i + 1])
        n = s1 - s0
        if n == 0:
            continue
        L = int(context_lens[i])
        assert n <= L, "more new tokens than context positions"
        kc_bits, vc_bits = gather_context(k_log, v_log, block_tables[i], L, block_size, num_blocks)
        kc = bits_to_f64(kc_bits, dtype)        # [L, Hkv, D]
        vc = bits_to_f64(vc_bits, dtype)
        qi = bits_to_f64(q[s0:s1], dtype)       # [n, Hq, D]
        for j in range(n):
            seen = visible_keys(position_of(L, n, j))
            for g in range(num_kv_heads):
                heads = [h for h in range(Hq) if kv_head_of(h, G) == g]
                out[s0 + j, heads] = attend(qi[j, heads], kc[:seen, g, :], vc[:seen, g, :], scale64)
    return out

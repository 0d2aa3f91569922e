"""Paged decode attention, from its definition (oracle; test infrastructure).

What is computed, for one decode step ("vLLM — PagedAttention으로 ...", section
"Prefill vs Decode": one new token per step, attending over the cached K/V of
every earlier token):

1. Gather.  Sequence i's logical block j lives in physical block
   block_tables[i, j] (same page, section "PagedAttention — OS 가상 메모리에서
   영감": logical blocks mapped onto non-contiguous physical ones; section
   "프로젝트 구조": the block manager keeps that mapping).  Token t of the context
   is token t mod bs of logical block t div bs.
2. Scores and softmax.  out = softmax(scale * q K^T) V over the L_i context
   tokens ("[Hacker News 요약] ... 'Tiny-vLLM' 직접 구축하기", section "고성능 추론을
   위한 고급 최적화 기법": the attention formula of "Attention is all you need",
   softmax normalisation, a causal mask keeping earlier tokens only).
3. GQA (same section): several q heads share one kv head.

Readings taken where the pages are silent:
* grouping order: q head h uses kv head h // G with G = Hq / Hkv (consecutive
  q heads share a kv head);
* the context length L_i counts the token appended this step (append first,
  then attend over positions 0 .. L_i - 1);
* the causal mask: the query is the last position, so the mask is t < L_i;
* L_i = 0 gives a zero output;
* table entries past ceil(L_i / bs) and tail slots of the last block are never
  read (the oracle asserts the first);
* the scale reaches the kernel as fp32, so the oracle uses float64(float32(scale)).

Everything is float64; the only library primitives are numpy's matrix-vector
product, exp and sum.  No blocking, splitting or online softmax.
"""
import numpy as np

from .layout import check_shape, k_logical, v_logical
from .numerics import bits_to_f64, scale_as_passed


def kv_head_of(h: int, group: int) -> int:
    """kv head read by q head h (contiguous grouping)."""
    return h // group


def gather_context(k_log, v_log, table_row, length, block_size, num_blocks):
    """Contiguous [L, Hkv, D] copies (still uint16 bits) of one sequence's K and V."""
    t = np.arange(length)
    logical_block = t // block_size
    phys = np.asarray(table_row, dtype=np.int64)[logical_block]
    assert np.all((phys >= 0) & (phys < num_blocks)), "block table entry out of range"
    off = t % block_size
    return k_log[phys, :, off, :], v_log[phys, :, off, :]


def attend(q_heads, k_ctx, v_ctx, scale64):
    """softmax(scale * q K^T) V for a [G, D] group of queries over [L, D] keys/values."""
    s = scale64 * (q_heads @ k_ctx.T)            # [G, L]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)                             # softmax numerator; max subtracted for range
    return (w @ v_ctx) / w.sum(axis=1, keepdims=True)


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, *, dtype, num_blocks,
           num_kv_heads, block_size, seqs=None):
    """Paged decode attention in float64.

    q: uint16 bits [B, Hq, D]; k_cache, v_cache: uint16 bits, flat physical pools of
    N*Hkv*bs*D elements in the layout of ``oracle.layout``; block_tables: int [B, M];
    context_lens: int [B].  Returns float64 [len(seqs), Hq, D] (all sequences if
    seqs is None).
    """
    q = np.asarray(q)
    B, Hq, D = q.shape
    check_shape(num_kv_heads, block_size, D)
    if Hq % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // num_kv_heads
    k_log = k_logical(np.asarray(k_cache), num_blocks, num_kv_heads, block_size, D)
    v_log = v_logical(np.asarray(v_cache), num_blocks, num_kv_heads, block_size, D)
    scale64 = scale_as_passed(scale)
    seqs = range(B) if seqs is None else list(seqs)
    out = np.zeros((len(seqs), Hq, D), dtype=np.float64)
    for r, i in enumerate(seqs):
        L = int(context_lens[i])
        if L == 0:
            continue
        kc_bits, vc_bits = gather_context(k_log, v_log, block_tables[i], L, block_size, num_blocks)
        kc = bits_to_f64(kc_bits, dtype)        # [L, Hkv, D]
        vc = bits_to_f64(vc_bits, dtype)
        qi = bits_to_f64(q[i], dtype)           # [Hq, D]
        for g in range(num_kv_heads):
            heads = [h for h in range(Hq) if kv_head_of(h, G) == g]
            out[r, heads] = attend(qi[heads], kc[:, g, :], vc[:, g, :], scale64)
    return out

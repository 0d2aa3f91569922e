"""Scalar-loop reference for tiny cases (oracle; test infrastructure).

The same definition as ``oracle.attention`` (attention over the gathered
context with GQA, per the Tiny-vLLM summary page's section "고성능 추론을 위한
고급 최적화 기법"; paging per the vLLM page's section "PagedAttention — OS 가상
메모리에서 영감"), written as plain Python loops with math.exp and math.fsum and
reading each element through the offset formula, not the array view.  Meant for
contexts of a few dozen tokens and head dims of 8-16.
"""
import math

import numpy as np

from .layout import k_offset, v_offset
from .numerics import bits_to_f64, scale_as_passed


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, *, dtype, num_kv_heads, block_size):
    qf = bits_to_f64(np.asarray(q), dtype)
    kf = bits_to_f64(np.asarray(k_cache), dtype)
    vf = bits_to_f64(np.asarray(v_cache), dtype)
    B, Hq, D = qf.shape
    G = Hq // num_kv_heads
    sc = scale_as_passed(scale)
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    for i in range(B):
        L = int(context_lens[i])
        for h in range(Hq):
            g = h // G
            if L == 0:
                continue
            keys, vals = [], []
            for t in range(L):
                n = int(block_tables[i][t // block_size])
                off = t % block_size
                keys.append([kf[k_offset(n, g, off, d, num_kv_heads, block_size, D)] for d in range(D)])
                vals.append([vf[v_offset(n, g, off, d, num_kv_heads, block_size, D)] for d in range(D)])
            s = [sc * math.fsum(qf[i, h, d] * keys[t][d] for d in range(D)) for t in range(L)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            for d in range(D):
                out[i][h][d] = math.fsum(w[t] * vals[t][d] for t in range(L)) / z
    return np.array(out, dtype=np.float64)

"""Continuous-batching decode loop, replayed from its definition (oracle; test infrastructure).

Requests join and leave the running batch between token-generation iterations
("vLLM -- PagedAttention으로 LLM 추론 성능을 2~4배 끌어올린 서빙 엔진", section
"Continuous Batching"); where a sequence's blocks sit in the pool does not
change what it attends to (same page, section "PagedAttention -- OS 가상
메모리에서 영감").  So the replay keeps no pool and no block table: in each layer
a sequence's context is simply its prompt's K/V followed by the K/V appended at
each of its decode steps, in order, and a step's output for a sequence is the
attention of that step's q over the whole context (oracle.attention.attend,
float64, GQA grouping h // G).

Only tests import this module.
"""
import numpy as np

from .attention import attend, kv_head_of
from .numerics import bits_to_f64, scale_as_passed


class LoopReplay:
    def __init__(self, num_q_heads, num_kv_heads, head_dim, dtype, scale):
        if num_q_heads % num_kv_heads:
            raise ValueError("num_q_heads must be a multiple of num_kv_heads")
        self.Hq, self.Hkv, self.D = num_q_heads, num_kv_heads, head_dim
        self.G = num_q_heads // num_kv_heads
        self.dtype = dtype
        self.scale64 = scale_as_passed(scale)
        self.k = {}  # (rid, layer) -> uint16 bits [L, Hkv, D]
        self.v = {}

    def admit(self, rid, layer, k_prompt, v_prompt):
        """A new sequence whose context in `layer` starts with the prompt's K/V bits [P, Hkv, D]."""
        self.k[(rid, layer)] = np.asarray(k_prompt, dtype=np.uint16).reshape(-1, self.Hkv, self.D).copy()
        self.v[(rid, layer)] = np.asarray(v_prompt, dtype=np.uint16).reshape(-1, self.Hkv, self.D).copy()

    def step(self, layer, run_ids, q, k_new, v_new):
        """Append k_new[i] / v_new[i] to sequence run_ids[i]'s context, then attend with q[i].

        Returns float64 [B, Hq, D]."""
        out = np.zeros((len(run_ids), self.Hq, self.D), dtype=np.float64)
        for i, rid in enumerate(run_ids):
            key = (rid, layer)
            self.k[key] = np.concatenate([self.k[key], np.asarray(k_new[i], dtype=np.uint16)[None]], axis=0)
            self.v[key] = np.concatenate([self.v[key], np.asarray(v_new[i], dtype=np.uint16)[None]], axis=0)
            kc = bits_to_f64(self.k[key], self.dtype)
            vc = bits_to_f64(self.v[key], self.dtype)
            qi = bits_to_f64(q[i], self.dtype)
            for g in range(self.Hkv):
                heads = [h for h in range(self.Hq) if kv_head_of(h, self.G) == g]
                out[i, heads] = attend(qi[heads], kc[:, g, :], vc[:, g, :], self.scale64)
        return out

    def context(self, rid, layer):
        """The K and V bits [L, Hkv, D] of a sequence's context in one layer."""
        return self.k[(rid, layer)], self.v[(rid, layer)]

    def finish(self, rid, num_layers):
        for layer in range(num_layers):
            self.k.pop((rid, layer), None)
            self.v.pop((rid, layer), None)

"""Seeded request streams and step plans for a continuous-batching decode loop.

Continuous batching, as the pages describe it: requests join and leave the
running batch at every token-generation iteration instead of the whole batch
waiting for its slowest member ("vLLM -- PagedAttention으로 LLM 추론 성능을 2~4배
끌어올린 서빙 엔진", section "Continuous Batching"; the Tiny-vLLM summary, section
"고성능 추론을 위한 고급 최적화 기법", lists it among the serving techniques).

This module only decides *what* happens at each step -- which requests are
admitted, which sequences decode, which finish -- and draws the values (prompt
K/V, and each step's q and appended k/v).  It holds none of the attention
arithmetic; the GPU loop and the oracle replay both consume its plans.

Policy (the pages give none; the plainest one that never needs preemption):
first come, first served; a request is admitted when the batch has room and
the pool can hold the blocks the request will ever need, ceil((P + G) / bs)
for a P-token prompt and G generated tokens.  An admitted request's prompt K/V
is written into the cache (there is no model, so a prompt is just its K/V);
then every running sequence decodes one token per step -- the token's K/V is
appended and its query attends over the whole context, prompt included -- and
a sequence leaves after its G-th step.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Tuple

import numpy as np

from . import BF16, random_bits


@dataclasses.dataclass(frozen=True)
class LoopConfig:
    name: str
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    num_blocks: int        # blocks in each layer's pool
    max_batch: int         # most sequences decoding at once
    num_requests: int
    prompt_lo: int         # prompt lengths: uniform [lo, hi], or lognormal with mean `prompt_mean`, clipped
    prompt_hi: int
    gen_lo: int            # generated tokens per request, likewise
    gen_hi: int
    lengths: str = "uniform"  # "uniform" | "lognormal"
    prompt_mean: float = 0.0
    gen_mean: float = 0.0
    arrivals_per_step: float = 0.0  # 0: every request is waiting at step 0
    prefix_groups: int = 0          # > 0: request r's prompt starts with group (r mod groups)'s
    prefix_tokens: int = 0          #      prefix of this many tokens (prompts are given as token ids)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def max_context(self) -> int:
        return self.prompt_hi + self.gen_hi


LOOP_CONFIGS = {
    # small enough that the fp64 oracle replays every step in seconds
    "tiny-loop": LoopConfig("tiny-loop", 2, 8, 2, 64, 16, BF16, num_blocks=48, max_batch=6, num_requests=14,
                            prompt_lo=1, prompt_hi=70, gen_lo=1, gen_hi=24, arrivals_per_step=0.8),
    # the same loop with prompts made of token ids, requests in 3 groups sharing a 40-token
    # prefix (two full blocks and a partial one), for prefix caching
    "tiny-prefix-loop": LoopConfig("tiny-prefix-loop", 2, 8, 2, 64, 16, BF16, num_blocks=48, max_batch=6,
                                   num_requests=14, prompt_lo=1, prompt_hi=70, gen_lo=1, gen_hi=24,
                                   arrivals_per_step=0.8, prefix_groups=3, prefix_tokens=40),
    # Llama-3.2-1B attention shape (16 layers, 32 q / 8 kv heads, head_dim 64, bs 16, bf16) with the
    # length mix of the 256-sequence continuous-batching workload (lognormal, mean 600); a backlog of
    # requests keeps the batch full
    "cb-llama3.2-1b": LoopConfig("cb-llama3.2-1b", 16, 32, 8, 64, 16, BF16, num_blocks=20480, max_batch=256,
                                 num_requests=4096, prompt_lo=1, prompt_hi=8000, gen_lo=1, gen_hi=1024,
                                 lengths="lognormal", prompt_mean=600.0, gen_mean=128.0),
}


@dataclasses.dataclass(frozen=True)
class Request:
    rid: int
    arrival: int
    prompt_len: int
    gen_len: int


@dataclasses.dataclass
class Step:
    index: int
    admit: List[int]    # request ids admitted before this step's decode (prompt written)
    run: List[int]      # request ids decoding this step, in batch order (ascending id)
    finish: List[int]   # request ids that leave after this step


def _lognormal(rng, mean, lo, hi, n):
    x = rng.lognormal(mean=math.log(mean) - 0.5, sigma=1.0, size=n)
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def requests(lc: LoopConfig, seed: int) -> List[Request]:
    """The request stream: arrival step, prompt length, tokens to generate."""
    rng = np.random.default_rng([seed, 0])
    n = lc.num_requests
    if lc.lengths == "lognormal":
        prompt = _lognormal(rng, lc.prompt_mean, lc.prompt_lo, lc.prompt_hi, n)
        gen = _lognormal(rng, lc.gen_mean, lc.gen_lo, lc.gen_hi, n)
    else:
        prompt = rng.integers(lc.prompt_lo, lc.prompt_hi + 1, size=n)
        gen = rng.integers(lc.gen_lo, lc.gen_hi + 1, size=n)
    if lc.arrivals_per_step > 0:
        arrival = np.cumsum(rng.poisson(1.0 / lc.arrivals_per_step, size=n)) - 1
        arrival = np.maximum(arrival, 0)
    else:
        arrival = np.zeros(n, dtype=np.int64)
    return [Request(i, int(arrival[i]), int(prompt[i]), int(gen[i])) for i in range(n)]


def blocks_for(tokens: int, block_size: int) -> int:
    return -(-tokens // block_size)


def plan(lc: LoopConfig, seed: int, num_steps: int) -> Tuple[List[Request], List[Step]]:
    """The first num_steps steps of the loop under the admission policy above."""
    reqs = requests(lc, seed)
    waiting = list(reqs)             # in arrival order (ids ascend with arrival)
    running = {}                     # rid -> tokens generated so far
    reserved = 0
    steps = []
    for s in range(num_steps):
        admitted = []
        while waiting and waiting[0].arrival <= s and len(running) < lc.max_batch:
            r = waiting[0]
            need = blocks_for(r.prompt_len + r.gen_len, lc.block_size)
            if reserved + need > lc.num_blocks:
                break
            waiting.pop(0)
            reserved += need
            running[r.rid] = 0
            admitted.append(r.rid)
        run = sorted(running)
        finish = []
        for rid in run:
            running[rid] += 1
            if running[rid] == reqs[rid].gen_len:
                finish.append(rid)
        for rid in finish:
            del running[rid]
            reserved -= blocks_for(reqs[rid].prompt_len + reqs[rid].gen_len, lc.block_size)
        steps.append(Step(s, admitted, run, finish))
    return reqs, steps


def prompt_tokens(lc: LoopConfig, seed: int, rid: int, prompt_len: int) -> np.ndarray:
    """Token ids of request rid's prompt (int32 [P]): its group's prefix, then its own tokens."""
    own = np.random.default_rng([seed, 3, rid]).integers(0, 32000, size=prompt_len).astype(np.int32)
    if lc.prefix_groups <= 0:
        return own
    pre = np.random.default_rng([seed, 4, rid % lc.prefix_groups]).integers(0, 32000, size=lc.prefix_tokens)
    n = min(prompt_len, lc.prefix_tokens)
    own[:n] = pre[:n]
    return own


def token_values(lc: LoopConfig, seed: int, tokens, layer: int):
    """K and V bits [P, Hkv, D] of a prompt given as token ids, where row t depends only on
    tokens[0..t] (as a model's keys and values do), so equal prefixes give equal rows."""
    P = len(tokens)
    k = np.empty((P, lc.num_kv_heads, lc.head_dim), dtype=np.uint16)
    v = np.empty_like(k)
    h = 0
    for t in range(P):
        h = (h * 1000003 + int(tokens[t]) + 1) % (1 << 61)
        rng = np.random.default_rng([seed, 5, layer, h])
        k[t] = random_bits(rng, (lc.num_kv_heads, lc.head_dim), lc.dtype)
        v[t] = random_bits(rng, (lc.num_kv_heads, lc.head_dim), lc.dtype)
    return k, v


def prompt_values(lc: LoopConfig, seed: int, rid: int, layer: int, prompt_len: int):
    """K and V bits of request rid's prompt in one layer: uint16 [P, Hkv, D] each."""
    rng = np.random.default_rng([seed, 1, rid, layer])
    shape = (prompt_len, lc.num_kv_heads, lc.head_dim)
    return random_bits(rng, shape, lc.dtype), random_bits(rng, shape, lc.dtype)


def step_values(lc: LoopConfig, seed: int, step: int, layer: int, batch: int):
    """q [B, Hq, D], and the appended k and v [B, Hkv, D] of one step in one layer (uint16 bits)."""
    rng = np.random.default_rng([seed, 2, step, layer])
    q = random_bits(rng, (batch, lc.num_q_heads, lc.head_dim), lc.dtype)
    k = random_bits(rng, (batch, lc.num_kv_heads, lc.head_dim), lc.dtype)
    v = random_bits(rng, (batch, lc.num_kv_heads, lc.head_dim), lc.dtype)
    return q, k, v

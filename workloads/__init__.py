"""Seeded synthetic inputs for paged decode attention and the KV append.

This module only builds inputs: context lengths, a shuffled physical block
pool dealt out into per-sequence block tables, random q/K/V values, the slot
of each appended token, and the slots/blocks that parity runs poison with NaN.
It holds none of the attention arithmetic and knows nothing about how a
(block, head, token, dim) element is placed inside a block: it only relies on
the cache being an array whose outermost dimension is the physical block, so
that block n is the flat range [n*E, (n+1)*E) with E = Hkv*bs*D elements.

Both the CPU oracle and the GPU path take their inputs from here; neither side
is imported by this module.

The five workloads follow the shapes the pages talk about: a tiny two-sequence
case; a Llama-3.2-1B-shaped decode batch (bf16, 32 q heads / 8 kv heads /
head_dim 64; the Tiny-vLLM page names that model and bf16); a long-context batch
with 256-token blocks (the block size the Nano-vLLM page gives as default); one
LLaMA-2-70B-shaped fp16 layer (80 layers, 64 heads, head_dim 128, 4096 tokens in
the vLLM page's KV-size example, here one layer of it); and a continuous-batching
step over 16 layers with a shared 512-token prompt prefix (prefix caching on the
Nano-vLLM page).  All values are N(0,1) drawn in fp32 and rounded to the
storage type; nothing is taken from a dataset.

Draw order per workload (one numpy Generator seeded with the workload seed):
context lengths, block permutation, then per layer q, K pool, V pool, appended
k, appended v.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

BF16 = "bf16"
FP16 = "fp16"

NAN_BITS = {BF16: 0x7FC0, FP16: 0x7E00}


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    num_layers: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    lengths: str          # "fixed" | "uniform" | "lognormal"
    len_lo: int = 0
    len_hi: int = 0
    fixed_lens: tuple = ()
    pool_blocks: int = 0  # 0 = sized to fit the total
    prefix_groups: int = 0
    prefix_blocks: int = 0

    @property
    def scale(self) -> float:
        """1/sqrt(head_dim), as fp32."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 2


CONFIGS = {
    1: Config(1, "tiny", 1, 2, 4, 2, 64, 16, BF16, "fixed", fixed_lens=(5, 37), pool_blocks=16),
    2: Config(2, "llama3.2-1b-b64", 1, 64, 32, 8, 64, 16, BF16, "uniform", 128, 2048),
    3: Config(3, "long-context-b16", 1, 16, 32, 8, 64, 256, BF16, "uniform", 4096, 8192),
    4: Config(4, "llama2-70b-layer-mha", 1, 8, 64, 64, 128, 16, FP16, "fixed", fixed_lens=(4096,) * 8),
    5: Config(5, "cb-step-16l-b256", 16, 256, 32, 8, 64, 16, BF16, "lognormal", 1, 8192,
              prefix_groups=8, prefix_blocks=32),
}


def f32_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to bf16/fp16 (round to nearest even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == FP16:
        return x.astype(np.float16).view(np.uint16)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def random_bits(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return f32_to_bits(rng.standard_normal(shape, dtype=np.float32), dtype)


@dataclasses.dataclass
class Layer:
    q: np.ndarray        # uint16 [B, Hq, D]
    k_cache: np.ndarray  # uint16 flat, N*Hkv*bs*D elements, block-major
    v_cache: np.ndarray  # uint16 flat, same size
    k_new: np.ndarray    # uint16 [B, Hkv, D]: the token appended this step
    v_new: np.ndarray


@dataclasses.dataclass
class Workload:
    cfg: Config
    seed: int
    context_lens: np.ndarray   # int32 [B]; includes the token appended this step
    block_tables: np.ndarray   # int32 [B, max_blocks]; padded with pad_block
    num_blocks: int
    pad_block: int             # a block no sequence uses (NaN-filled in parity runs)
    slot_mapping: np.ndarray   # int64 [B]: slot of position L_i - 1
    tail_slots: np.ndarray     # int64: slots of positions >= L_i inside each last block
    unused_blocks: np.ndarray  # int64: physical blocks referenced by no sequence
    shared_blocks: np.ndarray  # int64 [groups, prefix_blocks] (empty unless cfg 5)
    layers: List[Layer]

    @property
    def max_blocks(self) -> int:
        return self.block_tables.shape[1]

    @property
    def block_elems(self) -> int:
        c = self.cfg
        return c.num_kv_heads * c.block_size * c.head_dim


def _draw_lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    if cfg.lengths == "fixed":
        return np.asarray(cfg.fixed_lens, dtype=np.int64)
    if cfg.lengths == "uniform":
        return rng.integers(cfg.len_lo, cfg.len_hi + 1, size=cfg.num_seqs).astype(np.int64)
    # lognormal with mean 600: mu = ln(600) - sigma^2/2, sigma = 1, rounded, clipped
    x = rng.lognormal(mean=math.log(600.0) - 0.5, sigma=1.0, size=cfg.num_seqs)
    return np.clip(np.rint(x), cfg.len_lo, cfg.len_hi).astype(np.int64)


def build(cid: int, *, seed: Optional[int] = None, **kw) -> Workload:
    """Build workload ``cid`` (seed defaults to the workload number)."""
    return build_config(CONFIGS[cid], seed=cid if seed is None else seed, **kw)


def custom(num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int, lengths,
           dtype: str = BF16, *, seed: int = 0, spare_blocks: int = 1, **kw) -> Workload:
    """A one-layer workload of any shape (used by tests for small and edge cases)."""
    cfg = Config(0, "custom", 1, len(lengths), num_q_heads, num_kv_heads, head_dim, block_size,
                 dtype, "fixed", fixed_lens=tuple(int(x) for x in lengths))
    need = sum(-(-int(x) // block_size) for x in lengths)
    cfg = dataclasses.replace(cfg, pool_blocks=need + max(spare_blocks, 1))
    return build_config(cfg, seed=seed, **kw)


def build_config(cfg: Config, *, seed: int, poison: bool = True,
                 num_layers: Optional[int] = None, lengths: Optional[np.ndarray] = None,
                 num_seqs: Optional[int] = None) -> Workload:
    """Build the inputs of ``cfg``.

    poison: fill unused physical blocks (including the padding block) with
        NaN.  Tail slots are returned in ``tail_slots`` for the caller to
        poison through each side's own append.
    num_layers / lengths / num_seqs: overrides used by tests for smaller cases.
    """
    if num_seqs is not None:
        cfg = dataclasses.replace(cfg, num_seqs=num_seqs)
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, D, bs = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    L = _draw_lengths(cfg, rng) if lengths is None else np.asarray(lengths, dtype=np.int64)
    B = len(L)
    nblk = (L + bs - 1) // bs

    # which logical blocks are shared prefix blocks (config 5 rule): logical block j
    # of sequence i uses its group's shared block j iff j < prefix_blocks and the
    # block is full and lies strictly before the appended token: bs*(j+1) <= L_i - 1.
    groups = cfg.prefix_groups
    shared_mask = np.zeros((B, int(nblk.max()) if B else 0), dtype=bool)
    if groups:
        per_group = B // groups
        for i in range(B):
            for j in range(min(cfg.prefix_blocks, int(nblk[i]))):
                if bs * (j + 1) <= L[i] - 1:
                    shared_mask[i, j] = True
    n_shared = groups * cfg.prefix_blocks
    n_private = int(nblk.sum() - shared_mask.sum())
    needed = n_shared + n_private
    if cfg.pool_blocks:
        N = cfg.pool_blocks
        assert N > needed, "pool too small"
    else:
        N = needed + 1  # one spare block serves as table padding
    perm = rng.permutation(N).astype(np.int64)

    shared = perm[:n_shared].reshape(groups, cfg.prefix_blocks) if groups else np.zeros((0, 0), np.int64)
    cursor = n_shared
    maxb = int(nblk.max()) if B else 1
    pad_block = int(perm[needed])  # first block after the used ones
    tables = np.full((B, max(maxb, 1)), pad_block, dtype=np.int32)
    for i in range(B):
        for j in range(int(nblk[i])):
            if groups and shared_mask[i, j]:
                tables[i, j] = shared[i // (B // groups), j]
            else:
                tables[i, j] = perm[cursor]
                cursor += 1
    assert cursor == needed
    used = set(perm[:needed].tolist())
    unused = np.array(sorted(set(range(N)) - used), dtype=np.int64)

    # slot of the appended token (position L_i - 1) and the tail slots
    # (positions L_i .. nblk_i*bs - 1 of the last block)
    slots = np.full(B, -1, dtype=np.int64)
    tails = []
    for i in range(B):
        if L[i] == 0:
            continue
        pos = L[i] - 1
        slots[i] = int(tables[i, pos // bs]) * bs + pos % bs
        last = int(tables[i, nblk[i] - 1])
        for off in range(int(L[i] - (nblk[i] - 1) * bs), bs):
            tails.append(last * bs + off)
    tails = np.asarray(tails, dtype=np.int64)

    nl = cfg.num_layers if num_layers is None else num_layers
    E = Hkv * bs * D
    layers = []
    for _ in range(nl):
        q = random_bits(rng, (B, Hq, D), cfg.dtype)
        kc = random_bits(rng, (N * E,), cfg.dtype)
        vc = random_bits(rng, (N * E,), cfg.dtype)
        kn = random_bits(rng, (B, Hkv, D), cfg.dtype)
        vn = random_bits(rng, (B, Hkv, D), cfg.dtype)
        if poison:
            nan = np.uint16(NAN_BITS[cfg.dtype])
            for n in unused:
                kc[n * E:(n + 1) * E] = nan
                vc[n * E:(n + 1) * E] = nan
        layers.append(Layer(q, kc, vc, kn, vn))

    return Workload(cfg=cfg, seed=seed, context_lens=L.astype(np.int32), block_tables=tables,
                    num_blocks=N, pad_block=pad_block, slot_mapping=slots, tail_slots=tails,
                    unused_blocks=unused, shared_blocks=shared, layers=layers)


def nan_tokens(n: int, cfg: Config) -> np.ndarray:
    """[n, Hkv, D] tokens whose every element is NaN (used to poison tail slots)."""
    return np.full((n, cfg.num_kv_heads, cfg.head_dim), NAN_BITS[cfg.dtype], dtype=np.uint16)

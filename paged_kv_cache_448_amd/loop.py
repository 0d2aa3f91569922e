"""Continuous-batching decode loop: the host block allocator driving the library's kernels.

Each step of a plan (requests admitted, sequences decoding, sequences leaving;
see workloads.loop for the plans used in tests and benchmarks):

1. the admitted requests take the blocks of their prompts from the host
   allocator -- sharing the full blocks of a prompt prefix that a live
   sequence already holds when the prompts come as token ids -- and the K/V of
   the prompt positions not already cached is written into each layer's pool
   (one kv_append per layer for all of them, one slot per token);
2. every running sequence takes the slot of its next token (append_slots: a
   fresh block whenever the last one is full), and the running batch's block
   tables, context lengths and slots are copied to the device with the step's
   plan: the prefix items of sequences whose tables start with the same blocks
   (pkv_decode_prefix_plan: such a prefix is read once per item) and, with
   prefix items, the live partitions of a split plan (pkv_decode_work_list);
   otherwise the dispatch order (pkv_decode_schedule: the XCDs get equal work,
   long contexts start first);
3. each layer runs one fused append + decode launch (and a merge when the plan
   splits or shares prefixes);
4. sequences that are done return their blocks to the pool.  Their blocks may
   be handed out again in the next step; the stream orders the next step's
   writes after this step's reads.

Host arrays go through a small ring of pinned buffers so the host can prepare
the next steps while the GPU runs the current one.  The per-step launches call
the C ABI directly with pointers checked once at construction (the pools, the
staging buffers) or by shape (the caller's q/k/v/out), because at hundreds of
sequences and 16 layers a step's host time is otherwise dominated by argument
checking.  Everything on the device path is the library's kernels.
"""
from __future__ import annotations

import ctypes
import math
import time

import numpy as np
import torch

from . import PKV_BF16, PKV_FP16, check, lib, new_cache
from ._lib import PkvError
from .allocator import BlockAllocator

_TORCH_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}
_DTYPE_CODES = {"bf16": PKV_BF16, "fp16": PKV_FP16}


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


class DecodeLoop:
    """Pools for every layer, the host allocator, and the per-step staging."""

    def __init__(self, lc, device="cuda", shuffle_seed: int = 1, ring: int = 4, max_prompt_tokens: int = 0,
                 schedule: bool = True):
        self.lc = lc
        self.device = torch.device(device)
        self.dtype = _TORCH_DTYPES[lc.dtype]
        self.code = _DTYPE_CODES[lc.dtype]
        self.alloc = BlockAllocator(lc.num_blocks, lc.block_size, shuffle_seed)
        self.k_pools = [new_cache(lc.num_blocks, lc.num_kv_heads, lc.block_size, lc.head_dim, self.dtype, self.device)
                        for _ in range(lc.num_layers)]
        self.v_pools = [new_cache(lc.num_blocks, lc.num_kv_heads, lc.block_size, lc.head_dim, self.dtype, self.device)
                        for _ in range(lc.num_layers)]
        self.max_blocks = math.ceil(lc.max_context / lc.block_size)
        # prompt tokens one step may admit (default: a full batch of the longest prompts)
        self.max_prompt_tokens = max_prompt_tokens if max_prompt_tokens > 0 else lc.max_batch * lc.prompt_hi
        B = lc.max_batch
        # covers every step's plan (the batch's longest context changes every step), shared
        # prefixes of any length included
        ws = int(lib().pkv_decode_prefix_workspace_bytes(B, lc.num_q_heads, lc.num_kv_heads, lc.head_dim,
                                                         lc.block_size, lc.max_context, lc.max_context, 0))
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=self.device)
        self.tables_d = torch.empty(B * self.max_blocks, dtype=torch.int32, device=self.device)
        self.lens_d = torch.empty(B, dtype=torch.int32, device=self.device)
        self.slots_d = torch.empty(B, dtype=torch.int64, device=self.device)
        self.schedule = schedule
        self.order_d = torch.empty(B, dtype=torch.int32, device=self.device)
        # per-step shared-prefix plan and work list of the live partitions (host-built)
        self.items_cap = B // 2 + 1
        self.pre_len_d = torch.empty(B, dtype=torch.int32, device=self.device)
        self.items_d = torch.empty(self.items_cap * 16, dtype=torch.int32, device=self.device)
        self.work_cap = 64 * B * lc.num_kv_heads
        self.work_d = torch.empty(2 * self.work_cap, dtype=torch.int32, device=self.device)
        self.prompt_slots_d = torch.empty(self.max_prompt_tokens, dtype=torch.int64, device=self.device)
        pin = dict(pin_memory=True)
        self._ring = [dict(tables=torch.empty(B * self.max_blocks, dtype=torch.int32, **pin),
                           lens=torch.empty(B, dtype=torch.int32, **pin),
                           slots=torch.empty(B, dtype=torch.int64, **pin),
                           order=torch.empty(B, dtype=torch.int32, **pin),
                           pslots=torch.empty(self.max_prompt_tokens, dtype=torch.int64, **pin),
                           pre_len=torch.empty(B, dtype=torch.int32, **pin),
                           items=torch.empty(self.items_cap * 16, dtype=torch.int32, **pin),
                           work=torch.empty(2 * self.work_cap, dtype=torch.int32, **pin),
                           done=None) for _ in range(ring)]
        self._next = 0
        self._lib = lib()
        self.host_wait_s = 0.0  # time the host spent waiting for the GPU to free a staging buffer
        self.prefix_steps = 0   # steps whose decode read shared prefixes once per prefix item

    def _staging(self):
        st = self._ring[self._next]
        self._next = (self._next + 1) % len(self._ring)
        if st["done"] is not None:
            t0 = time.perf_counter()
            st["done"].synchronize()  # the copies out of this buffer have run
            self.host_wait_s += time.perf_counter() - t0
        return st

    def _release(self, st, stream):
        ev = torch.cuda.Event()
        ev.record(stream)
        st["done"] = ev

    def _check(self, t, shape, name):
        if not (t.is_cuda and t.dtype == self.dtype and t.is_contiguous() and tuple(t.shape) == shape):
            raise PkvError(f"{name} must be a contiguous {self.dtype} GPU tensor of shape {shape}, got "
                           f"{t.dtype} {tuple(t.shape)}")

    def admit(self, rids, prompt_lens, prompt_kv, token_ids=None):
        """Register requests rids with their prompts and write the prompts' K/V.

        Without token_ids every prompt gets fresh blocks.  With token_ids (one int
        array per request) the allocator shares the leading full blocks that a live
        sequence already holds for the same tokens (prefix caching), and only the
        positions after them are written.  prompt_kv(layer, cached) -> (k, v): device
        tensors [T, Hkv, D] holding, request after request in the order of rids,
        positions cached[i] .. prompt_lens[i]-1 (T = the sum of those counts).
        Returns cached, the per-request count of prompt tokens already in the pool."""
        lc, bs = self.lc, self.lc.block_size
        cached, slots = [], []
        for i, (rid, P) in enumerate(zip(rids, prompt_lens)):
            P = int(P)
            if token_ids is None:
                self.alloc.add_seq(int(rid), P)
                c = 0
            else:
                if len(token_ids[i]) != P:
                    raise PkvError(f"request {rid}: {len(token_ids[i])} token ids for a {P}-token prompt")
                c = self.alloc.add_seq_prefix(int(rid), token_ids[i])
            cached.append(c)
            if P > c:
                table, _ = self.alloc.block_tables([int(rid)], -(-P // bs))
                pos = np.arange(c, P, dtype=np.int64)
                slots.append(table[0, pos // bs].astype(np.int64) * bs + pos % bs)
        T = int(sum(len(s) for s in slots))
        if T == 0:
            return cached
        if T > self.max_prompt_tokens:
            raise PkvError(f"{T} prompt tokens in one step; the loop stages at most {self.max_prompt_tokens}")
        stream = torch.cuda.current_stream(self.device)
        st = self._staging()
        st["pslots"][:T].numpy()[:] = np.concatenate(slots)
        self.prompt_slots_d[:T].copy_(st["pslots"][:T], non_blocking=True)
        self._release(st, stream)
        shape = (T, lc.num_kv_heads, lc.head_dim)
        sp = ctypes.c_void_p(stream.cuda_stream)
        for layer in range(lc.num_layers):
            k, v = prompt_kv(layer, cached)
            self._check(k, shape, "prompt k")
            self._check(v, shape, "prompt v")
            check(self._lib.pkv_kv_append(_p(k), _p(v), _p(self.prompt_slots_d), T, _p(self.k_pools[layer]),
                                          _p(self.v_pools[layer]), lc.num_blocks, bs, lc.num_kv_heads, lc.head_dim,
                                          self.code, sp))
        return cached

    def decode_step(self, run_ids, step_qkv, outs):
        """One token for every sequence in run_ids (batch order).

        step_qkv(layer) -> (q [B, Hq, D], k [B, Hkv, D], v [B, Hkv, D]) device tensors;
        outs[layer]: [B, Hq, D] output tensors.  Returns the batch's context lengths."""
        lc, bs = self.lc, self.lc.block_size
        B = len(run_ids)
        if B == 0:
            return np.zeros(0, dtype=np.int32)
        if B > lc.max_batch:
            raise PkvError(f"batch of {B} exceeds the loop's max_batch {lc.max_batch}")
        slots = self.alloc.append_slots(run_ids)
        tables, lens = self.alloc.block_tables(run_ids, self.max_blocks, pad_value=0)
        lens_max = int(lens.max())
        M = -(-lens_max // bs)  # only the columns the batch uses go to the device
        stream = torch.cuda.current_stream(self.device)
        st = self._staging()
        st["tables"][:B * M].numpy().reshape(B, M)[:] = tables[:, :M]
        st["lens"][:B].numpy()[:] = lens
        st["slots"][:B].numpy()[:] = slots
        self.tables_d[:B * M].copy_(st["tables"][:B * M], non_blocking=True)
        self.lens_d[:B].copy_(st["lens"][:B], non_blocking=True)
        self.slots_d[:B].copy_(st["slots"][:B], non_blocking=True)
        # Shared prefixes (blocks the allocator gave several sequences) are read once per
        # prefix item; a split plan launches only its live partitions.  Both are planned
        # here from the host's tables and lengths, outside the launches.
        items_n, max_pl = self._plan_prefixes(st, tables, lens, M)
        self.prefix_steps += items_n > 0
        # (without shared prefixes the full grid in dispatch order measured 2% faster on the
        # 256-sequence loop than the work list)
        work_n = self._plan_work(st, lens, lens_max, True) if items_n else 0
        order = None
        if self.schedule and work_n == 0:
            o = st["order"][:B].numpy()
            check(self._lib.pkv_decode_schedule(lens.ctypes.data, B, o.ctypes.data))
            self.order_d[:B].copy_(st["order"][:B], non_blocking=True)
            order = _p(self.order_d)
        self._release(st, stream)
        sp = ctypes.c_void_p(stream.cuda_stream)
        qs, kvs = (B, lc.num_q_heads, lc.head_dim), (B, lc.num_kv_heads, lc.head_dim)
        ws = ctypes.c_size_t(self.workspace.numel())
        scale = ctypes.c_float(lc.scale)
        pre = (_p(self.pre_len_d), _p(self.items_d)) if items_n else (None, None)
        work = _p(self.work_d) if work_n else None
        for layer in range(lc.num_layers):
            q, k, v = step_qkv(layer)
            out = outs[layer]
            self._check(q, qs, "q")
            self._check(k, kvs, "k")
            self._check(v, kvs, "v")
            self._check(out, qs, "out")
            check(self._lib.pkv_paged_attn_decode_prefix(
                _p(q), _p(k), _p(v), _p(self.slots_d), _p(self.k_pools[layer]), _p(self.v_pools[layer]),
                _p(self.tables_d), M, _p(self.lens_d), lens_max, scale, _p(out), B, lc.num_q_heads, lc.num_kv_heads,
                lc.head_dim, bs, lc.num_blocks, self.code, pre[0], pre[1], items_n, max_pl, _p(self.workspace), ws,
                0, order, work, work_n, sp))
        return lens

    def _plan_prefixes(self, st, tables, lens, M):
        """Prefix items of this step's batch (pkv_decode_prefix_plan) copied to the device;
        returns (items, longest prefix)."""
        lc, B = self.lc, len(lens)
        tab = np.ascontiguousarray(tables[:, :M])
        pl = st["pre_len"][:B].numpy()
        it = st["items"].numpy()
        n, longest = ctypes.c_int32(), ctypes.c_int32()
        check(self._lib.pkv_decode_prefix_plan(tab.ctypes.data, M, lens.ctypes.data, B, lc.num_q_heads,
                                               lc.num_kv_heads, lc.head_dim, lc.block_size, pl.ctypes.data,
                                               it.ctypes.data, self.items_cap, ctypes.byref(n), ctypes.byref(longest)))
        if n.value:
            self.pre_len_d[:B].copy_(st["pre_len"][:B], non_blocking=True)
            self.items_d[:16 * n.value].copy_(st["items"][:16 * n.value], non_blocking=True)
        return n.value, longest.value

    def _plan_work(self, st, lens, lens_max, prefixed):
        """The live partitions of a split plan (pkv_decode_work_list) copied to the device;
        0 when the plan is a single pass (the dispatch order is used then)."""
        lc, B = self.lc, len(lens)
        if self._lib.pkv_decode_plan_partition(B, lc.num_kv_heads, lc.block_size, lens_max) == 0:
            return 0
        pl = st["pre_len"][:B].numpy() if prefixed else None
        n = ctypes.c_int32()
        args = (lens.ctypes.data, None if pl is None else pl.ctypes.data, B, lc.num_kv_heads, lens_max, 0)
        status = self._lib.pkv_decode_work_list(*args, st["work"].numpy().ctypes.data, self.work_cap,
                                                ctypes.byref(n))
        if status != 0 and n.value > self.work_cap:
            # a larger list than any before: grow every staging buffer and the device copy
            self.work_cap = n.value
            for r in self._ring:
                if r["done"] is not None:
                    r["done"].synchronize()
                r["work"] = torch.empty(2 * n.value, dtype=torch.int32, pin_memory=True)
            self.work_d = torch.empty(2 * n.value, dtype=torch.int32, device=self.device)
            status = self._lib.pkv_decode_work_list(*args, st["work"].numpy().ctypes.data, self.work_cap,
                                                    ctypes.byref(n))
        check(status)
        self.work_d[:2 * n.value].copy_(st["work"][:2 * n.value], non_blocking=True)
        return n.value

    def finish(self, rid: int):
        self.alloc.free_seq(int(rid))

    def gather(self, rid: int, layer: int):
        """K and V of sequence rid in one layer, in token order, as device tensors [L, Hkv, D] (for checks)."""
        L = self.alloc.context_len(rid)
        bs = self.lc.block_size
        table, _ = self.alloc.block_tables([rid], max(1, -(-L // bs)))
        pos = torch.arange(L, device=self.device)
        blk = torch.from_numpy(table[0].astype(np.int64)).to(self.device)[pos // bs]
        k = self.k_pools[layer][blk, :, pos % bs, :]
        v = self.v_pools[layer][blk, :, pos % bs, :]
        return k, v

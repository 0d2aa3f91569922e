"""Paged KV-cache decode attention for AMD MI355X (gfx950).

Python binding of ``libpkv.so`` (ctypes).  It only marshals arguments: torch
tensors supply device memory and the current HIP stream, and every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing, every call raises.

Names mirror the C ABI in include/pkv.h and include/pkv_alloc.h:

* ``kv_append(k, v, slot_mapping, k_cache, v_cache)``
* ``paged_attn_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out)``
* ``append_paged_attn_decode(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
  context_lens, scale, out)`` -- both in one launch (one decode step of one layer)
* ``paged_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, out)`` --
  causal attention of the new tokens of every sequence (packed rows) over its paged context
* ``kv_append_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale)`` and
  ``paged_attn_decode_fp8(q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale, out)``
  -- the same over FP8 (E4M3) pools (uint8 tensors, see ``new_cache_fp8``)
* ``BlockAllocator`` -- the host-side block allocator.

Caches are tensors of shape ``(num_blocks, num_kv_heads, block_size, head_dim)``
(see ``new_cache``): one contiguous row of ``head_dim`` values per (block, kv
head, token of the block), K and V alike.
"""
import ctypes
import os

import numpy as np

import torch

from ._lib import PKV_BF16, PKV_FP16, PkvError, check, lib  # noqa: F401

__all__ = ["kv_append", "paged_attn_decode", "append_paged_attn_decode", "decode_workspace_bytes",
           "decode_supported", "plan_partition", "new_cache", "new_cache_fp8", "cache_dims", "kv_append_fp8",
           "paged_attn_decode_fp8", "paged_prefill", "decode_prefix_plan", "decode_prefix_workspace_bytes",
           "decode_work_list", "paged_attn_decode_prefix", "PrefixPlan", "BlockAllocator", "PkvError", "lib"]

_DTYPES = {torch.bfloat16: PKV_BF16, torch.float16: PKV_FP16}
IMPLS = {"auto": 0, "simt": 1, "mfma": 2}


def _dtype_code(t):
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise PkvError(f"unsupported dtype {t.dtype}; use bfloat16 or float16") from None


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(cond, msg):
    if not cond:
        raise PkvError(msg)


def _device_tensor(t, name, dtype=None, ndim=None):
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    _need(t.is_cuda, f"{name} must be on a GPU")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None:
        _need(t.dim() == ndim, f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")


def new_cache(num_blocks, num_kv_heads, block_size, head_dim, dtype=torch.bfloat16, device="cuda"):
    """Uninitialised K or V pool in the library's layout."""
    _need(block_size % 16 == 0, "block_size must be a multiple of 16")
    return torch.empty((num_blocks, num_kv_heads, block_size, head_dim), dtype=dtype, device=device)


def new_cache_fp8(num_blocks, num_kv_heads, block_size, head_dim, device="cuda"):
    """Uninitialised FP8 (E4M3 code per element) K or V pool in the library's layout."""
    return new_cache(num_blocks, num_kv_heads, block_size, head_dim, torch.uint8, device)


def cache_dims(cache):
    """(num_blocks, num_kv_heads, block_size, head_dim) of a pool made by new_cache."""
    _need(cache.dim() == 4 and cache.shape[2] % 16 == 0, f"bad cache shape {tuple(cache.shape)}")
    n, h, b, d = cache.shape
    return int(n), int(h), int(b), int(d)


def kv_append(k, v, slot_mapping, k_cache, v_cache):
    """Write k/v ([T, Hkv, D]) into the slots ``slot_mapping`` (int64 [T]) of the pools."""
    N, Hkv, bs, D = cache_dims(k_cache)
    _need(tuple(v_cache.shape) == tuple(k_cache.shape), "k_cache and v_cache differ in shape")
    for name, t in (("k", k), ("v", v)):
        _device_tensor(t, name, k_cache.dtype, 3)
        _need(tuple(t.shape[1:]) == (Hkv, D), f"{name} must be [T, {Hkv}, {D}], got {tuple(t.shape)}")
    _need(k.shape == v.shape, "k and v differ in shape")
    _device_tensor(slot_mapping, "slot_mapping", torch.int64, 1)
    _need(slot_mapping.shape[0] == k.shape[0], "slot_mapping must have one slot per token")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _device_tensor(t, name)
    check(lib().pkv_kv_append(_ptr(k), _ptr(v), _ptr(slot_mapping), k.shape[0], _ptr(k_cache), _ptr(v_cache),
                              N, bs, Hkv, D, _dtype_code(k_cache), _stream(k_cache)))


def decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                           partition_tokens=0):
    return int(lib().pkv_decode_workspace_bytes_ex(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                                   max_context_len, partition_tokens))


def decode_supported(impl, dtype, head_dim, group):
    """Whether decode kernel ``impl`` ("auto", "simt", "mfma") is built for these sizes."""
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else {"bf16": PKV_BF16, "fp16": PKV_FP16}[dtype]
    return bool(lib().pkv_decode_supported(IMPLS[impl], code, int(head_dim), int(group)))


def plan_partition(num_seqs, num_kv_heads, block_size, max_context_len):
    return int(lib().pkv_decode_plan_partition(num_seqs, num_kv_heads, block_size, max_context_len))


def decode_schedule(context_lens):
    """Dispatch order for the decode calls' ``seq_order``, from the host's copy of
    the context lengths (int sequence or numpy array): longest first, dealt so
    that the XCDs get about equal work.  Returns an int32 numpy permutation."""
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    _need(lens.ndim == 1, "context_lens must be one-dimensional")
    order = np.empty(lens.shape[0], dtype=np.int32)
    check(lib().pkv_decode_schedule(lens.ctypes.data, int(lens.shape[0]), order.ctypes.data))
    return order


def _order_ptr(seq_order, B):
    if seq_order is None:
        return None
    _device_tensor(seq_order, "seq_order", torch.int32, 1)
    _need(seq_order.shape[0] == B, "seq_order must have one entry per sequence")
    return _ptr(seq_order)


def paged_attn_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out=None, *,
                      max_context_len=None, workspace=None, partition_tokens=0, impl="auto", seq_order=None):
    """softmax(scale q K^T) V per sequence over its paged context.

    q: [B, Hq, D]; block_tables: int32 [B, M]; context_lens: int32 [B] (device);
    max_context_len: host-side bound of every length (default M * block_size);
    workspace: uint8 device tensor of at least decode_workspace_bytes(...) bytes
    (allocated through torch when omitted); seq_order: optional int32 [B] device
    permutation (see decode_schedule), which changes only the work order.
    Returns ``out`` ([B, Hq, D]).
    """
    N, Hkv, bs, D = cache_dims(k_cache)
    _need(tuple(v_cache.shape) == tuple(k_cache.shape), "k_cache and v_cache differ in shape")
    _device_tensor(q, "q", k_cache.dtype, 3)
    B, Hq, Dq = (int(x) for x in q.shape)
    _need(Dq == D, f"q head_dim {Dq} != cache head_dim {D}")
    _device_tensor(k_cache, "k_cache")
    _device_tensor(v_cache, "v_cache")
    _device_tensor(block_tables, "block_tables", torch.int32, 2)
    _need(block_tables.shape[0] == B, "block_tables must have one row per sequence")
    _device_tensor(context_lens, "context_lens", torch.int32, 1)
    _need(context_lens.shape[0] == B, "context_lens must have one entry per sequence")
    M = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = M * bs
    if out is None:
        out = torch.empty_like(q)
    else:
        _device_tensor(out, "out", q.dtype, 3)
        _need(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    need = decode_workspace_bytes(B, Hq, Hkv, D, bs, max_context_len, partition_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    else:
        _device_tensor(workspace, "workspace", torch.uint8)
    _need(impl in IMPLS, f"impl must be one of {sorted(IMPLS)}")
    check(lib().pkv_paged_attn_decode_ex(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), M, _ptr(context_lens), int(max_context_len),
        ctypes.c_float(scale), _ptr(out), B, Hq, Hkv, D, bs, N, _dtype_code(q), _ptr(workspace),
        ctypes.c_size_t(workspace.numel()), int(partition_tokens), IMPLS[impl], _order_ptr(seq_order, B),
        _stream(q)))
    return out


def paged_attn_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, out, *, max_context_len=None):
    """paged_attn_decode through the allocation-free entry point: no workspace, the
    split-context partial states in the library's per-GPU device array (calls that
    overlap on one GPU race).  ``out`` ([B, Hq, D], q's dtype) is required, so that
    nothing is allocated here either."""
    N, Hkv, bs, D = cache_dims(k_cache)
    _need(tuple(v_cache.shape) == tuple(k_cache.shape), "k_cache and v_cache differ in shape")
    _device_tensor(q, "q", k_cache.dtype, 3)
    B, Hq, Dq = (int(x) for x in q.shape)
    _need(Dq == D, f"q head_dim {Dq} != cache head_dim {D}")
    _device_tensor(k_cache, "k_cache")
    _device_tensor(v_cache, "v_cache")
    _device_tensor(block_tables, "block_tables", torch.int32, 2)
    _need(block_tables.shape[0] == B, "block_tables must have one row per sequence")
    _device_tensor(context_lens, "context_lens", torch.int32, 1)
    _need(context_lens.shape[0] == B, "context_lens must have one entry per sequence")
    _device_tensor(out, "out", q.dtype, 3)
    _need(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    M = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = M * bs
    check(lib().pkv_paged_attn_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), M, _ptr(context_lens), int(max_context_len),
        ctypes.c_float(scale), _ptr(out), B, Hq, Hkv, D, bs, N, _dtype_code(q), _stream(q)))
    return out


def append_paged_attn_decode(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, context_lens, scale,
                             out=None, *, max_context_len=None, workspace=None, partition_tokens=0, seq_order=None):
    """kv_append of one token per sequence, then paged_attn_decode, in one launch.

    k_new, v_new: [B, Hkv, D]; slot_mapping: int64 [B], the slot of position
    context_lens[i] - 1 of sequence i (negative: nothing appended for it).
    Same result as the two calls when that holds; a slot that is not that
    position's slot is not written and makes sequence i's output NaN.
    """
    N, Hkv, bs, D = cache_dims(k_cache)
    _need(tuple(v_cache.shape) == tuple(k_cache.shape), "k_cache and v_cache differ in shape")
    _device_tensor(q, "q", k_cache.dtype, 3)
    B, Hq, Dq = (int(x) for x in q.shape)
    _need(Dq == D, f"q head_dim {Dq} != cache head_dim {D}")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _device_tensor(t, name, k_cache.dtype, 3)
        _need(tuple(t.shape) == (B, Hkv, D), f"{name} must be [{B}, {Hkv}, {D}], got {tuple(t.shape)}")
    _device_tensor(slot_mapping, "slot_mapping", torch.int64, 1)
    _need(slot_mapping.shape[0] == B, "slot_mapping must have one slot per sequence")
    _device_tensor(k_cache, "k_cache")
    _device_tensor(v_cache, "v_cache")
    _device_tensor(block_tables, "block_tables", torch.int32, 2)
    _need(block_tables.shape[0] == B, "block_tables must have one row per sequence")
    _device_tensor(context_lens, "context_lens", torch.int32, 1)
    _need(context_lens.shape[0] == B, "context_lens must have one entry per sequence")
    M = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = M * bs
    if out is None:
        out = torch.empty_like(q)
    else:
        _device_tensor(out, "out", q.dtype, 3)
        _need(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    need = decode_workspace_bytes(B, Hq, Hkv, D, bs, max_context_len, partition_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    else:
        _device_tensor(workspace, "workspace", torch.uint8)
    check(lib().pkv_append_paged_attn_decode(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), M,
        _ptr(context_lens), int(max_context_len), ctypes.c_float(scale), _ptr(out), B, Hq, Hkv, D, bs, N,
        _dtype_code(q), _ptr(workspace), ctypes.c_size_t(workspace.numel()), int(partition_tokens),
        _order_ptr(seq_order, B), _stream(q)))
    return out


class PrefixPlan:
    """Shared-prefix work found by decode_prefix_plan: ``prefix_len`` (int32 [B]),
    ``items`` (int32 [num_items, 16], member 0 the reference, -1 pads) and
    ``max_prefix_len``, as host numpy arrays / ints."""

    def __init__(self, prefix_len, items, max_prefix_len):
        self.prefix_len = prefix_len
        self.items = items
        self.max_prefix_len = int(max_prefix_len)

    @property
    def num_items(self):
        return int(self.items.shape[0])


def decode_prefix_plan(block_tables, context_lens, num_q_heads, num_kv_heads, head_dim, block_size):
    """Group the sequences whose block tables start with the same blocks (host
    numpy int32 tables [B, M] and lengths [B]) into prefix items for
    paged_attn_decode_prefix.  Returns a PrefixPlan."""
    tables = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    _need(tables.ndim == 2 and lens.ndim == 1 and tables.shape[0] == lens.shape[0],
          "block_tables must be [B, M] and context_lens [B]")
    B, M = (int(x) for x in tables.shape)
    cap = B // 2 + 1
    prefix_len = np.zeros(B, dtype=np.int32)
    items = np.full((cap, 16), -1, dtype=np.int32)
    n = ctypes.c_int32()
    longest = ctypes.c_int32()
    check(lib().pkv_decode_prefix_plan(tables.ctypes.data, M, lens.ctypes.data, B, int(num_q_heads),
                                       int(num_kv_heads), int(head_dim), int(block_size), prefix_len.ctypes.data,
                                       items.ctypes.data, cap, ctypes.byref(n), ctypes.byref(longest)))
    return PrefixPlan(prefix_len, items[:n.value].copy(), longest.value)


def decode_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                                  max_prefix_len, partition_tokens=0):
    return int(lib().pkv_decode_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                                       max_context_len, max_prefix_len, partition_tokens))


def decode_work_list(context_lens, num_kv_heads, max_context_len, partition_tokens=0, prefix_len=None):
    """One entry per workgroup of a split decode's live work, from host lengths (and a
    PrefixPlan's prefix_len), dealt over the XCDs: int32 numpy [n, 2] of (sequence,
    partition | kv head << 16 | one-wave-per-head << 31); sequence -1 pads."""
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    _need(lens.ndim == 1, "context_lens must be one-dimensional")
    B = int(lens.shape[0])
    pl = None
    if prefix_len is not None:
        pl = np.ascontiguousarray(np.asarray(prefix_len, dtype=np.int32))
        _need(pl.shape == lens.shape, "prefix_len must have one entry per sequence")
    args = (lens.ctypes.data, None if pl is None else pl.ctypes.data, B, int(num_kv_heads), int(max_context_len),
            int(partition_tokens))
    n = ctypes.c_int32()
    status = lib().pkv_decode_work_list(*args, None, 0, ctypes.byref(n))  # the size needed
    if status != 0 and n.value == 0:
        check(status)
    work = np.empty((max(n.value, 1), 2), dtype=np.int32)
    check(lib().pkv_decode_work_list(*args, work.ctypes.data, work.shape[0], ctypes.byref(n)))
    return work[:n.value].copy()


def paged_attn_decode_prefix(q, k_cache, v_cache, block_tables, context_lens, scale, prefix_len, prefix_items,
                             max_prefix_len, out=None, *, k_new=None, v_new=None, slot_mapping=None,
                             max_context_len=None, workspace=None, partition_tokens=0, seq_order=None, work=None):
    """paged_attn_decode (MFMA kernel) with shared prefixes read once per prefix item,
    optionally with the step's append fused in (k_new, v_new, slot_mapping as in
    append_paged_attn_decode).

    prefix_len: int32 [B] and prefix_items: int32 [n, 16], device copies of a
    PrefixPlan's arrays; max_prefix_len: its host bound.  work: optional int32
    [n, 2] device copy of decode_work_list's output for the same arguments.
    """
    N, Hkv, bs, D = cache_dims(k_cache)
    _need(tuple(v_cache.shape) == tuple(k_cache.shape), "k_cache and v_cache differ in shape")
    _device_tensor(q, "q", k_cache.dtype, 3)
    B, Hq, Dq = (int(x) for x in q.shape)
    _need(Dq == D, f"q head_dim {Dq} != cache head_dim {D}")
    fused = slot_mapping is not None
    if fused:
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            _device_tensor(t, name, k_cache.dtype, 3)
            _need(tuple(t.shape) == (B, Hkv, D), f"{name} must be [{B}, {Hkv}, {D}], got {tuple(t.shape)}")
        _device_tensor(slot_mapping, "slot_mapping", torch.int64, 1)
        _need(slot_mapping.shape[0] == B, "slot_mapping must have one slot per sequence")
    _device_tensor(k_cache, "k_cache")
    _device_tensor(v_cache, "v_cache")
    _device_tensor(block_tables, "block_tables", torch.int32, 2)
    _need(block_tables.shape[0] == B, "block_tables must have one row per sequence")
    _device_tensor(context_lens, "context_lens", torch.int32, 1)
    _need(context_lens.shape[0] == B, "context_lens must have one entry per sequence")
    _device_tensor(prefix_len, "prefix_len", torch.int32, 1)
    _need(prefix_len.shape[0] == B, "prefix_len must have one entry per sequence")
    _device_tensor(prefix_items, "prefix_items", torch.int32, 2)
    _need(prefix_items.shape[1] == 16, "prefix_items must be [n, 16]")
    M = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = M * bs
    if out is None:
        out = torch.empty_like(q)
    else:
        _device_tensor(out, "out", q.dtype, 3)
        _need(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    need = decode_prefix_workspace_bytes(B, Hq, Hkv, D, bs, max_context_len, max_prefix_len, partition_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    else:
        _device_tensor(workspace, "workspace", torch.uint8)
    check(lib().pkv_paged_attn_decode_prefix(
        _ptr(q), _ptr(k_new) if fused else None, _ptr(v_new) if fused else None,
        _ptr(slot_mapping) if fused else None, _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), M,
        _ptr(context_lens), int(max_context_len), ctypes.c_float(scale), _ptr(out), B, Hq, Hkv, D, bs, N,
        _dtype_code(q), _ptr(prefix_len), _ptr(prefix_items), int(prefix_items.shape[0]), int(max_prefix_len),
        _ptr(workspace), ctypes.c_size_t(workspace.numel()), int(partition_tokens), _order_ptr(seq_order, B),
        _work_ptr(work), 0 if work is None else int(work.shape[0]), _stream(q)))
    return out


def _work_ptr(work):
    if work is None:
        return None
    _device_tensor(work, "work", torch.int32, 2)
    _need(work.shape[1] == 2, "work must be [n, 2]")
    return _ptr(work)


def paged_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, out=None, *,
                  max_query_len, max_context_len=None):
    """Causal attention of the new tokens of every sequence over its paged context.

    q: [T, Hq, D], sequence i's new tokens at rows query_start[i] .. query_start[i+1]-1
    (query_start: int32 [B + 1] on the device); context_lens: int32 [B], each L_i
    counting the new tokens, which are the last n_i positions; max_query_len: host
    bound of every n_i; max_context_len: host bound of every L_i (default M * block_size).
    Returns ``out`` ([T, Hq, D])."""
    N, Hkv, bs, D = cache_dims(k_cache)
    _need(tuple(v_cache.shape) == tuple(k_cache.shape), "k_cache and v_cache differ in shape")
    _device_tensor(q, "q", k_cache.dtype, 3)
    T, Hq, Dq = (int(x) for x in q.shape)
    _need(Dq == D, f"q head_dim {Dq} != cache head_dim {D}")
    _device_tensor(k_cache, "k_cache")
    _device_tensor(v_cache, "v_cache")
    _device_tensor(block_tables, "block_tables", torch.int32, 2)
    B = int(block_tables.shape[0])
    _device_tensor(context_lens, "context_lens", torch.int32, 1)
    _need(context_lens.shape[0] == B, "context_lens must have one entry per sequence")
    _device_tensor(query_start, "query_start", torch.int32, 1)
    _need(query_start.shape[0] == B + 1, "query_start must have num_seqs + 1 entries")
    M = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = M * bs
    if out is None:
        out = torch.empty_like(q)
    else:
        _device_tensor(out, "out", q.dtype, 3)
        _need(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    check(lib().pkv_paged_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), M, _ptr(context_lens),
                                  _ptr(query_start), T, int(max_query_len), int(max_context_len), ctypes.c_float(scale),
                                  _ptr(out), B, Hq, Hkv, D, bs, N, _dtype_code(q), _stream(q)))
    return out


def _scale(x, name):
    x = float(x)
    _need(x > 0 and x < float("inf"), f"{name} must be positive and finite, got {x}")
    return ctypes.c_float(x)


def kv_append_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale):
    """Quantise k/v ([T, Hkv, D], bf16 or fp16) to E4M3 codes of x / scale and write them
    into the slots ``slot_mapping`` (int64 [T]) of the uint8 pools."""
    N, Hkv, bs, D = cache_dims(k_cache)
    _need(tuple(v_cache.shape) == tuple(k_cache.shape), "k_cache and v_cache differ in shape")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _device_tensor(t, name, torch.uint8)
    _device_tensor(k, "k", None, 3)
    code = _dtype_code(k)
    for name, t in (("k", k), ("v", v)):
        _device_tensor(t, name, k.dtype, 3)
        _need(tuple(t.shape[1:]) == (Hkv, D), f"{name} must be [T, {Hkv}, {D}], got {tuple(t.shape)}")
    _need(k.shape == v.shape, "k and v differ in shape")
    _device_tensor(slot_mapping, "slot_mapping", torch.int64, 1)
    _need(slot_mapping.shape[0] == k.shape[0], "slot_mapping must have one slot per token")
    check(lib().pkv_kv_append_fp8(_ptr(k), _ptr(v), _ptr(slot_mapping), k.shape[0], _ptr(k_cache), _ptr(v_cache),
                                  N, bs, Hkv, D, code, _scale(k_scale, "k_scale"), _scale(v_scale, "v_scale"),
                                  _stream(k_cache)))


def paged_attn_decode_fp8(q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale, out=None, *,
                          max_context_len=None, workspace=None, partition_tokens=0, seq_order=None):
    """paged_attn_decode over FP8 pools: K = e4m3(k_cache) * k_scale, V = e4m3(v_cache) * v_scale.

    q (bf16 or fp16) [B, Hq, D]; the pools are uint8 tensors from new_cache_fp8;
    the other arguments as paged_attn_decode.  Returns ``out`` ([B, Hq, D], q's dtype).
    """
    N, Hkv, bs, D = cache_dims(k_cache)
    _need(tuple(v_cache.shape) == tuple(k_cache.shape), "k_cache and v_cache differ in shape")
    _device_tensor(k_cache, "k_cache", torch.uint8)
    _device_tensor(v_cache, "v_cache", torch.uint8)
    _device_tensor(q, "q", None, 3)
    code = _dtype_code(q)
    B, Hq, Dq = (int(x) for x in q.shape)
    _need(Dq == D, f"q head_dim {Dq} != cache head_dim {D}")
    _device_tensor(block_tables, "block_tables", torch.int32, 2)
    _need(block_tables.shape[0] == B, "block_tables must have one row per sequence")
    _device_tensor(context_lens, "context_lens", torch.int32, 1)
    _need(context_lens.shape[0] == B, "context_lens must have one entry per sequence")
    M = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = M * bs
    if out is None:
        out = torch.empty_like(q)
    else:
        _device_tensor(out, "out", q.dtype, 3)
        _need(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    need = decode_workspace_bytes(B, Hq, Hkv, D, bs, max_context_len, partition_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    else:
        _device_tensor(workspace, "workspace", torch.uint8)
    check(lib().pkv_paged_attn_decode_fp8(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), M, _ptr(context_lens), int(max_context_len),
        ctypes.c_float(scale), _scale(k_scale, "k_scale"), _scale(v_scale, "v_scale"), _ptr(out), B, Hq, Hkv, D, bs,
        N, code, _ptr(workspace), ctypes.c_size_t(workspace.numel()), int(partition_tokens),
        _order_ptr(seq_order, B), _stream(q)))
    return out


def append_paged_attn_decode_fp8(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, context_lens, scale,
                                 k_scale, v_scale, out=None, *, max_context_len=None, workspace=None,
                                 partition_tokens=0, seq_order=None):
    """kv_append_fp8 of one token per sequence, then paged_attn_decode_fp8, in one launch.

    k_new, v_new: [B, Hkv, D] in q's dtype; slot_mapping: int64 [B], the slot of
    position context_lens[i] - 1 of sequence i (negative: nothing appended).
    Same pools and output as the two calls when that holds; a slot that is not
    that position's slot is not written and makes sequence i's output NaN.
    """
    N, Hkv, bs, D = cache_dims(k_cache)
    _need(tuple(v_cache.shape) == tuple(k_cache.shape), "k_cache and v_cache differ in shape")
    _device_tensor(k_cache, "k_cache", torch.uint8)
    _device_tensor(v_cache, "v_cache", torch.uint8)
    _device_tensor(q, "q", None, 3)
    code = _dtype_code(q)
    B, Hq, Dq = (int(x) for x in q.shape)
    _need(Dq == D, f"q head_dim {Dq} != cache head_dim {D}")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _device_tensor(t, name, q.dtype, 3)
        _need(tuple(t.shape) == (B, Hkv, D), f"{name} must be [{B}, {Hkv}, {D}], got {tuple(t.shape)}")
    _device_tensor(slot_mapping, "slot_mapping", torch.int64, 1)
    _need(slot_mapping.shape[0] == B, "slot_mapping must have one slot per sequence")
    _device_tensor(block_tables, "block_tables", torch.int32, 2)
    _need(block_tables.shape[0] == B, "block_tables must have one row per sequence")
    _device_tensor(context_lens, "context_lens", torch.int32, 1)
    _need(context_lens.shape[0] == B, "context_lens must have one entry per sequence")
    M = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = M * bs
    if out is None:
        out = torch.empty_like(q)
    else:
        _device_tensor(out, "out", q.dtype, 3)
        _need(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    need = decode_workspace_bytes(B, Hq, Hkv, D, bs, max_context_len, partition_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    else:
        _device_tensor(workspace, "workspace", torch.uint8)
    check(lib().pkv_append_paged_attn_decode_fp8(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), M,
        _ptr(context_lens), int(max_context_len), ctypes.c_float(scale), _scale(k_scale, "k_scale"),
        _scale(v_scale, "v_scale"), _ptr(out), B, Hq, Hkv, D, bs, N, code, _ptr(workspace),
        ctypes.c_size_t(workspace.numel()), int(partition_tokens), _order_ptr(seq_order, B), _stream(q)))
    return out


from .allocator import BlockAllocator  # noqa: E402

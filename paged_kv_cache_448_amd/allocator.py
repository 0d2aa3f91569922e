"""Python handle for the host-side block allocator (include/pkv_alloc.h)."""
import ctypes

import numpy as np

from ._lib import PkvError, check, lib


class BlockAllocator:
    """Free list + reference counts over a pool of ``num_blocks`` KV blocks.

    Produces block tables, context lengths and the slot of each appended token
    as numpy arrays; the caller moves them to the device.  Not thread-safe.
    """

    def __init__(self, num_blocks: int, block_size: int, shuffle_seed: int = 0):
        self._h = lib().pkv_alloc_create(int(num_blocks), int(block_size), ctypes.c_uint64(shuffle_seed))
        if not self._h:
            raise PkvError("pkv_alloc_create failed (bad sizes or out of memory)")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self):
        if self._h:
            lib().pkv_alloc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_seq(self, seq_id: int, num_tokens: int):
        check(lib().pkv_alloc_add_seq(self._h, int(seq_id), int(num_tokens)))

    def add_seq_shared(self, seq_id: int, num_tokens: int, src_seq: int, num_shared_blocks: int):
        check(lib().pkv_alloc_add_seq_shared(self._h, int(seq_id), int(num_tokens), int(src_seq),
                                             int(num_shared_blocks)))

    def share_prefix(self, dst_seq: int, src_seq: int, num_full_blocks: int):
        """Make dst_seq's first num_full_blocks blocks src_seq's (both live; the blocks full and
        before both sequences' next write); dst_seq's own blocks there are released."""
        check(lib().pkv_alloc_share_prefix(self._h, int(dst_seq), int(src_seq), int(num_full_blocks)))

    def add_seq_prefix(self, seq_id: int, token_ids) -> int:
        """Register seq_id with its prompt's token ids, sharing the leading full blocks that
        the pool still holds for the same tokens (held by a live sequence, or freed but not yet
        reused); returns how many leading tokens' K/V are already in the pool (the caller
        writes K/V only for the rest)."""
        ids = np.ascontiguousarray(token_ids, dtype=np.int32)
        out = ctypes.c_int32()
        check(lib().pkv_alloc_add_seq_prefix(self._h, int(seq_id), ids.ctypes.data if len(ids) else None, len(ids),
                                             ctypes.byref(out)))
        return out.value

    def append_slot(self, seq_id: int) -> int:
        out = ctypes.c_int64()
        check(lib().pkv_alloc_append_slot(self._h, int(seq_id), ctypes.byref(out)))
        return out.value

    def append_slots(self, seq_ids) -> np.ndarray:
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        out = np.empty(len(ids), dtype=np.int64)
        check(lib().pkv_alloc_append_slots(self._h, ids.ctypes.data, len(ids), out.ctypes.data))
        return out

    def free_seq(self, seq_id: int):
        check(lib().pkv_alloc_free_seq(self._h, int(seq_id)))

    def block_tables(self, seq_ids, max_blocks: int, pad_value: int = 0):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tables = np.empty((len(ids), int(max_blocks)), dtype=np.int32)
        lens = np.empty(len(ids), dtype=np.int32)
        check(lib().pkv_alloc_block_tables(self._h, ids.ctypes.data, len(ids), int(max_blocks), int(pad_value),
                                           tables.ctypes.data, lens.ctypes.data))
        return tables, lens

    @property
    def num_free(self) -> int:
        return int(lib().pkv_alloc_num_free(self._h))

    @property
    def num_cached(self) -> int:
        """Free blocks that still hold a registered prompt block (counted in num_free too)."""
        return int(lib().pkv_alloc_num_cached(self._h))

    @property
    def num_seqs(self) -> int:
        return int(lib().pkv_alloc_num_seqs(self._h))

    def context_len(self, seq_id: int) -> int:
        out = ctypes.c_int32()
        check(lib().pkv_alloc_context_len(self._h, int(seq_id), ctypes.byref(out)))
        return out.value

    def refcount(self, block: int) -> int:
        return int(lib().pkv_alloc_refcount(self._h, int(block)))

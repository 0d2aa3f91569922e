"""The KV append: scatter of new tokens' K/V into their cache slots (oracle; test infrastructure).

New K/V are written only into the blocks a sequence holds, as tokens arrive
("vLLM — PagedAttention으로 ...", section "PagedAttention — OS 가상 메모리에서
영감"; "KV Cache가 왜 병목인가": K and V of every past token are kept so they are
not recomputed).

Readings where the pages are silent: a slot is physical_block * bs + offset; a
negative slot means "padding token, skip"; slots must be distinct and below
N * bs (asserted); the copy is bit-for-bit, so every other bit of the cache is
left as it was.
"""
import numpy as np

from .layout import check_shape, k_offset, v_offset


def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, *, num_blocks, block_size):
    """Write k_new/v_new (uint16 [T, Hkv, D]) into the flat uint16 pools, in place."""
    k_new = np.asarray(k_new, dtype=np.uint16)
    v_new = np.asarray(v_new, dtype=np.uint16)
    T, Hkv, D = k_new.shape
    check_shape(Hkv, block_size, D)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    assert slots.shape == (T,)
    live = slots[slots >= 0]
    assert np.all(live < num_blocks * block_size), "slot beyond the pool"
    assert len(np.unique(live)) == len(live), "duplicate slot"
    h = np.arange(Hkv)[:, None]
    d = np.arange(D)[None, :]
    for t in range(T):
        s = int(slots[t])
        if s < 0:
            continue
        n, off = divmod(s, block_size)
        k_cache[k_offset(n, h, off, d, Hkv, block_size, D)] = k_new[t]
        v_cache[v_offset(n, h, off, d, Hkv, block_size, D)] = v_new[t]

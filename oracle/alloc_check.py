"""Validity of block tables and slots produced by a block allocator (oracle; test infrastructure).

Paging semantics ("vLLM — PagedAttention으로 ...", section "PagedAttention — OS
가상 메모리에서 영감", including its diagram; section "프로젝트 구조" for the block
manager): a sequence holds exactly as many fixed-size blocks as its tokens need,
blocks may be anywhere in the pool, blocks nobody holds are free for other
requests.  Shared prompt prefixes reuse the same blocks ("Nano-vLLM로 배우는
...", section "KV 캐시와 Block Manager").

Many assignments are correct, so this checks properties, not block ids:
* entries [0, ceil(L_i/bs)) of row i are valid block ids, the rest are padding;
* a physical block appears in at most one (sequence, logical index) place,
  unless it is declared shared, and then every use is at the same logical index
  and is a full block lying before the position the sequence writes next (so an
  append never writes into a shared block);
* the number of free blocks is N minus the distinct blocks in use;
* the slot of position p of sequence i is table[i, p // bs] * bs + p % bs.
"""
import numpy as np


def blocks_needed(length: int, block_size: int) -> int:
    return -(-int(length) // block_size)


def check_tables(tables, lens, *, num_blocks, block_size, pad_value, shared=(), appended=True):
    """appended: the lengths count a token appended this step (position L-1 was just
    written, so a shared block must end before it); False: the state right after a
    prompt is registered, whose next write is position L (a shared block must be full)."""
    tables = np.asarray(tables)
    lens = np.asarray(lens)
    shared = set(int(x) for x in shared)
    seen = {}
    for i in range(len(lens)):
        nb = blocks_needed(lens[i], block_size)
        row = tables[i]
        assert nb <= len(row), f"seq {i}: table too short"
        for j in range(nb):
            p = int(row[j])
            assert 0 <= p < num_blocks, f"seq {i} block {j}: id {p} out of range"
            if p in seen:
                assert p in shared, f"block {p} held twice but not shared"
                assert seen[p] == j, f"shared block {p} at different logical indices"
            seen[p] = j
            if p in shared:
                last = lens[i] - 1 if appended else lens[i]
                assert block_size * (j + 1) <= last, f"seq {i}: shared block {p} not full before the next write"
        assert np.all(row[nb:] == pad_value), f"seq {i}: padding entries wrong"
    return len(seen)


def free_count(tables, lens, *, num_blocks, block_size):
    used = set()
    for i in range(len(lens)):
        for j in range(blocks_needed(lens[i], block_size)):
            used.add(int(tables[i][j]))
    return num_blocks - len(used)


def slot_of(tables, seq, pos, block_size):
    return int(tables[seq][pos // block_size]) * block_size + pos % block_size

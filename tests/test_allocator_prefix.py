"""Prefix caching in the host allocator (pkv_alloc_add_seq_prefix), host only.

Pinned against a brute-force reading of the page's rule ("Nano-vLLM로 배우는
...", section "KV 캐시와 Block Manager": full blocks of a shared prompt prefix
are found by hash and reused): a new prompt shares exactly as many leading full
blocks as the longest full-block prefix it has in common with the prompt of a
live sequence -- a model that never hashes anything -- and the tables stay valid
(oracle.alloc_check, shared blocks declared).
"""
import numpy as np
import pytest

import paged_kv_cache_448_amd as pkv
from oracle import alloc_check

BS = 16


def _blocks(*names, tail=0, rng=None):
    """A prompt made of named 16-token blocks (same name = same tokens) and a partial tail."""
    toks = []
    for n in names:
        toks += [1000 * n + i for i in range(BS)]
    toks += [7 + i for i in range(tail)]
    return np.array(toks, dtype=np.int32)


def test_identical_prompts_share_full_blocks():
    a = pkv.BlockAllocator(64, BS, shuffle_seed=3)
    p = _blocks(1, 2, 3, tail=5)
    assert a.add_seq_prefix(10, p) == 0
    assert a.add_seq_prefix(11, p) == 3 * BS
    t, lens = a.block_tables([10, 11], 4, pad_value=-1)
    assert list(t[0, :3]) == list(t[1, :3]) and t[0, 3] != t[1, 3]
    for b in t[0, :3]:
        assert a.refcount(int(b)) == 2
    alloc_check.check_tables(t, lens, num_blocks=64, block_size=BS, pad_value=-1, shared=t[0, :3], appended=False)
    assert a.num_free == 64 - 5


def test_divergence_stops_sharing():
    a = pkv.BlockAllocator(64, BS, shuffle_seed=1)
    a.add_seq_prefix(0, _blocks(1, 2, 3))
    assert a.add_seq_prefix(1, _blocks(1, 2, 9)) == 2 * BS
    assert a.add_seq_prefix(2, _blocks(4, 2, 3)) == 0           # first block differs: nothing after it counts
    p = _blocks(1, 2, 3)
    p[BS + 3] += 1                                              # one token of block 1 differs
    assert a.add_seq_prefix(3, p) == BS


def test_partial_blocks_are_never_shared_and_appends_go_to_fresh_blocks():
    a = pkv.BlockAllocator(32, BS)
    p = _blocks(5, tail=9)
    a.add_seq_prefix(0, p)
    assert a.add_seq_prefix(1, p) == BS
    full = _blocks(5, 6)
    a.add_seq_prefix(2, full)
    assert a.add_seq_prefix(3, full) == 2 * BS                  # the whole prompt is cached
    t, _ = a.block_tables([2, 3], 3, pad_value=-1)
    s = a.append_slot(3)                                        # position 32 of sequence 3
    t3, _ = a.block_tables([3], 3, pad_value=-1)
    assert s // BS == t3[0, 2] and a.refcount(int(t3[0, 2])) == 1
    assert t3[0, 2] not in set(t[0, :2].tolist())


def test_registry_follows_the_holders():
    a = pkv.BlockAllocator(32, BS)
    a.add_seq_prefix(0, _blocks(1, 2))
    a.add_seq_prefix(1, _blocks(1, 3))        # shares block "1", registers its own "3"
    a.free_seq(0)                             # "1" still held by sequence 1; "2" is gone
    assert a.add_seq_prefix(2, _blocks(1, 2)) == BS
    assert a.add_seq_prefix(3, _blocks(1, 3)) == 2 * BS
    for s in (1, 2, 3):
        a.free_seq(s)
    assert a.num_free == 32
    assert a.add_seq_prefix(4, _blocks(1, 3)) == 0          # nothing live holds those tokens any more


def test_nomem_changes_nothing():
    a = pkv.BlockAllocator(4, BS)
    a.add_seq_prefix(0, _blocks(1, 2, 3))
    with pytest.raises(pkv.PkvError):
        a.add_seq_prefix(1, _blocks(1, 2, 4, 5))            # needs 2 fresh blocks, 1 free
    assert a.num_free == 1 and a.num_seqs == 1
    assert a.add_seq_prefix(1, _blocks(1, 2, 3, tail=3)) == 3 * BS


def _common_full_blocks(p, q):
    n = min(len(p), len(q)) // BS
    k = 0
    while k < n and np.array_equal(p[k * BS:(k + 1) * BS], q[k * BS:(k + 1) * BS]):
        k += 1
    return k


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_brute_force_model(seed):
    """Random admissions and frees over prompts built from a small alphabet of blocks."""
    rng = np.random.default_rng(seed)
    N = 400
    a = pkv.BlockAllocator(N, BS, shuffle_seed=seed + 1)
    live = {}
    next_id = 0
    for _ in range(300):
        if live and rng.random() < 0.35:
            sid = int(rng.choice(list(live)))
            a.free_seq(sid)
            del live[sid]
            continue
        names = [int(x) for x in rng.integers(0, 3, size=rng.integers(0, 6))]
        p = _blocks(*names, tail=int(rng.integers(0, BS)))
        want = max([_common_full_blocks(p, q) for q in live.values()], default=0)
        try:
            got = a.add_seq_prefix(next_id, p)
        except pkv.PkvError:
            continue
        assert got == want * BS, (got, want)
        live[next_id] = p
        next_id += 1
        ids = sorted(live)
        if ids:
            M = max(1, max(-(-len(live[i]) // BS) for i in ids))
            t, lens = a.block_tables(ids, M, pad_value=-1)
            used = [int(b) for i in range(len(ids)) for b in t[i, :-(-int(lens[i]) // BS)]]
            shared = {b for b in used if used.count(b) > 1}
            alloc_check.check_tables(t, lens, num_blocks=N, block_size=BS, pad_value=-1, shared=shared, appended=False)
            assert a.num_free == N - len(set(used))

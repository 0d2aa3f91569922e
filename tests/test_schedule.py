"""The host dispatch schedule (pkv_decode_schedule), without a GPU.

The order only decides which workgroup decodes which sequence, so what is
checked is that it is a permutation, that it balances the token totals of the
eight contiguous XCD groups, and that each group starts with its longest
context.  The pages fix what decode computes, not this order; the GPU tests
check that outputs with and without it are bit-identical."""
import numpy as np
import pytest

import paged_kv_cache_448_amd as pkv
import workloads
from paged_kv_cache_448_amd import PkvError

XCDS = 8


def _groups(order):
    B = len(order)
    base, extra = divmod(B, XCDS)
    out, k = [], 0
    for g in range(XCDS):
        n = base + (1 if g < extra else 0)
        out.append(list(order[k:k + n]))
        k += n
    return out


@pytest.mark.parametrize("B,seed", [(64, 2), (256, 5), (10, 1), (7, 3), (1, 0), (129, 4)])
def test_schedule_is_a_balanced_longest_first_permutation(B, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 4096, size=B).astype(np.int32)
    order = pkv.decode_schedule(lens)
    assert order.dtype == np.int32 and sorted(order.tolist()) == list(range(B))
    groups = _groups(order)
    for g in groups:
        gl = [int(lens[s]) for s in g]
        assert gl == sorted(gl, reverse=True), "a group does not start with its longest context"
    if B >= XCDS:
        sums = [sum(int(lens[s]) for s in g) for g in groups]
        # greedy dealing keeps every total within one context of every other
        assert max(sums) - min(sums) <= int(lens.max())


def test_schedule_balances_the_llama_batch():
    """On the Llama-3.2-1B batch (64 sequences, lengths 128..2048) the XCD groups'
    totals come within 3% of each other (the batch in its own order: 6,726 to
    10,787 tokens per group of 8)."""
    cfg = workloads.CONFIGS[2]
    lens = workloads._draw_lengths(cfg, np.random.default_rng(2)).astype(np.int32)
    plain = [int(lens[8 * g:8 * g + 8].sum()) for g in range(XCDS)]
    order = pkv.decode_schedule(lens)
    sums = [sum(int(lens[s]) for s in g) for g in _groups(order)]
    assert max(plain) / min(plain) > 1.5
    assert max(sums) / min(sums) < 1.03, sums


def test_schedule_edge_cases():
    assert pkv.decode_schedule(np.zeros(0, np.int32)).shape == (0,)
    # equal lengths: any permutation is balanced; ties keep index order inside a group
    order = pkv.decode_schedule(np.full(16, 100, np.int32))
    assert sorted(order.tolist()) == list(range(16))
    for g in _groups(order):
        assert g == sorted(g)
    # negative lengths (invalid sequences) count as empty and still get a slot
    order = pkv.decode_schedule(np.array([5, -3, 9, 0], np.int32))
    assert sorted(order.tolist()) == [0, 1, 2, 3]
    assert pkv.lib().pkv_decode_schedule(None, 3, None) == -1
    assert pkv.lib().pkv_decode_schedule(None, -1, None) == -2
    with pytest.raises(PkvError):
        pkv.check(pkv.lib().pkv_decode_schedule(None, 2, None))

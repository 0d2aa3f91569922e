"""The seeded input generators (host logic, CPU only)."""
import numpy as np

import workloads
from oracle import alloc_check


def test_tiny_config_matches_its_description():
    wl = workloads.build(1)
    assert list(wl.context_lens) == [5, 37]
    assert wl.num_blocks == 16
    assert len(wl.unused_blocks) == 12
    assert wl.block_tables.shape == (2, 3)
    perm = np.random.default_rng(1).permutation(16)
    assert wl.block_tables[0, 0] == perm[0]
    assert list(wl.block_tables[1]) == list(perm[1:4])


def test_deterministic_per_seed():
    a = workloads.build(2)
    b = workloads.build(2)
    assert np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.layers[0].k_cache, b.layers[0].k_cache)
    c = workloads.build(2, seed=99)
    assert not np.array_equal(a.context_lens, c.context_lens)


def test_uniform_lengths_in_range():
    wl = workloads.build(2, poison=False)
    assert wl.context_lens.min() >= 128 and wl.context_lens.max() <= 2048
    assert wl.num_blocks == int(((wl.context_lens + 15) // 16).sum()) + 1
    alloc_check.check_tables(wl.block_tables, wl.context_lens, num_blocks=wl.num_blocks, block_size=16,
                             pad_value=wl.pad_block)


def test_prefix_sharing_rule():
    wl = workloads.build(5, num_layers=1, poison=False)
    L = wl.context_lens
    assert L.min() >= 1 and L.max() <= 8192
    shared = wl.shared_blocks
    assert shared.shape == (8, 32)
    alloc_check.check_tables(wl.block_tables, L, num_blocks=wl.num_blocks, block_size=16,
                             pad_value=wl.pad_block, shared=shared.ravel())
    for i in range(256):
        g = i // 32
        nb = -(-int(L[i]) // 16)
        for j in range(min(32, nb)):
            is_shared = 16 * (j + 1) <= L[i] - 1
            assert (wl.block_tables[i, j] == shared[g, j]) == is_shared
    # the appended slot is never inside a shared block
    assert not np.isin(wl.slot_mapping // 16, shared.ravel()).any()


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1.0 + 2**-8 + 2**-20], dtype=np.float32)
    bits = workloads.f32_to_bits(x, "bf16")
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert list(back) == [1.0, 1.0, 1.0 + 2**-6, -2.5, 1.0 + 2**-7]


def test_tail_slots_cover_last_block_remainder():
    wl = workloads.custom(4, 2, 64, 16, [5, 16, 17], seed=0)
    assert len(wl.tail_slots) == 11 + 0 + 15

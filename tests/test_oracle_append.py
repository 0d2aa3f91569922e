"""The append oracle and the two statements of the cache layout (CPU only)."""
import numpy as np
import pytest

import oracle
import workloads
from oracle import layout


@pytest.mark.parametrize("Hkv,bs,D", [(2, 16, 64), (1, 32, 8), (3, 256, 16), (2, 16, 128)])
def test_offset_formula_matches_view(Hkv, bs, D):
    """Writing each element's logical index through the offset formula and reading
    it back through the reshape view gives the identity -- and the offsets are a
    permutation of the pool."""
    N = 3
    n, h, t, d = np.meshgrid(np.arange(N), np.arange(Hkv), np.arange(bs), np.arange(D), indexing="ij")
    logical_index = ((n * Hkv + h) * bs + t) * D + d
    ko = layout.k_offset(n, h, t, d, Hkv, bs, D).ravel()
    vo = layout.v_offset(n, h, t, d, Hkv, bs, D).ravel()
    assert np.array_equal(np.sort(ko), np.arange(N * Hkv * bs * D))
    assert np.array_equal(np.sort(vo), np.arange(N * Hkv * bs * D))
    kflat = np.empty(N * Hkv * bs * D, dtype=np.int64)
    vflat = np.empty_like(kflat)
    kflat[ko] = logical_index.ravel()
    vflat[vo] = logical_index.ravel()
    assert np.array_equal(layout.k_logical(kflat, N, Hkv, bs, D), logical_index)
    assert np.array_equal(layout.v_logical(vflat, N, Hkv, bs, D), logical_index)


def test_token_rows_are_contiguous():
    """K and V alike: one token's D values for one kv head are one contiguous row; rows of a
    block's tokens follow each other, then the next kv head, then the next block."""
    for off in (layout.k_offset, layout.v_offset):
        assert off(0, 0, 0, 1, 1, 16, 64) == 1
        assert off(0, 0, 1, 0, 1, 16, 64) == 64
        assert off(0, 1, 0, 0, 2, 16, 64) == 16 * 64
        assert off(1, 0, 0, 0, 2, 16, 64) == 2 * 16 * 64
        assert off(2, 1, 15, 63, 2, 16, 64) == ((2 * 2 + 1) * 16 + 15) * 64 + 63


def _case():
    wl = workloads.custom(4, 2, 64, 16, [5, 37, 16], seed=3, spare_blocks=3)
    return wl, wl.layers[0]


def test_append_round_trip_and_untouched_bits():
    wl, ly = _case()
    kc, vc = ly.k_cache.copy(), ly.v_cache.copy()
    oracle.kv_append(ly.k_new, ly.v_new, wl.slot_mapping, kc, vc, num_blocks=wl.num_blocks, block_size=16)
    K = layout.k_logical(kc, wl.num_blocks, 2, 16, 64)
    V = layout.v_logical(vc, wl.num_blocks, 2, 16, 64)
    for i, s in enumerate(wl.slot_mapping):
        n, off = divmod(int(s), 16)
        assert np.array_equal(K[n, :, off, :], ly.k_new[i])
        assert np.array_equal(V[n, :, off, :], ly.v_new[i])
    changed_k = np.flatnonzero(kc != ly.k_cache)
    K0 = layout.k_logical(ly.k_cache, wl.num_blocks, 2, 16, 64)
    # only elements of appended slots may differ
    mask = np.zeros_like(K0, dtype=bool)
    for s in wl.slot_mapping:
        n, off = divmod(int(s), 16)
        mask[n, :, off, :] = True
    Kchanged = K != K0
    assert not np.any(Kchanged & ~mask)
    assert len(changed_k) <= mask.sum()


def test_append_idempotent_and_order_free():
    wl, ly = _case()
    a_k, a_v = ly.k_cache.copy(), ly.v_cache.copy()
    oracle.kv_append(ly.k_new, ly.v_new, wl.slot_mapping, a_k, a_v, num_blocks=wl.num_blocks, block_size=16)
    b_k, b_v = a_k.copy(), a_v.copy()
    oracle.kv_append(ly.k_new, ly.v_new, wl.slot_mapping, b_k, b_v, num_blocks=wl.num_blocks, block_size=16)
    assert np.array_equal(a_k, b_k) and np.array_equal(a_v, b_v)
    p = np.array([2, 0, 1])
    c_k, c_v = ly.k_cache.copy(), ly.v_cache.copy()
    oracle.kv_append(ly.k_new[p], ly.v_new[p], wl.slot_mapping[p], c_k, c_v, num_blocks=wl.num_blocks,
                     block_size=16)
    assert np.array_equal(a_k, c_k) and np.array_equal(a_v, c_v)


def test_negative_slot_skipped_and_bad_slots_rejected():
    wl, ly = _case()
    kc, vc = ly.k_cache.copy(), ly.v_cache.copy()
    slots = wl.slot_mapping.copy()
    slots[1] = -1
    oracle.kv_append(ly.k_new, ly.v_new, slots, kc, vc, num_blocks=wl.num_blocks, block_size=16)
    K = layout.k_logical(kc, wl.num_blocks, 2, 16, 64)
    K0 = layout.k_logical(ly.k_cache, wl.num_blocks, 2, 16, 64)
    n, off = divmod(int(wl.slot_mapping[1]), 16)
    assert np.array_equal(K[n, :, off], K0[n, :, off])
    with pytest.raises(AssertionError):
        dup = wl.slot_mapping.copy()
        dup[1] = dup[0]
        oracle.kv_append(ly.k_new, ly.v_new, dup, kc, vc, num_blocks=wl.num_blocks, block_size=16)
    with pytest.raises(AssertionError):
        big = wl.slot_mapping.copy()
        big[0] = wl.num_blocks * 16
        oracle.kv_append(ly.k_new, ly.v_new, big, kc, vc, num_blocks=wl.num_blocks, block_size=16)

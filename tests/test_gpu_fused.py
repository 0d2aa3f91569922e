"""append_paged_attn_decode (kv_append + decode in one launch) on the GPU.

Against the two-call path (kv_append, then paged_attn_decode with the MFMA
kernel) on the same inputs: the pools must be bit-identical and the outputs
bit-identical; against the fp64 oracle the output must be within
|err| <= 1e-2 + 1e-2 |ref|.  Before the fused call the append slots are filled
with NaN, so a read of the slot's old contents instead of the new token would
show up as NaN.
"""
import functools

import numpy as np
import pytest
import torch

import paged_kv_cache_448_amd as pkv
import workloads
from gpu_harness import (assert_parity, gpu_decode, oracle_caches, oracle_decode, poison_tails_gpu, to_bits, to_dev,
                         upload)
from oracle.numerics import bits_to_f64

pytestmark = pytest.mark.gpu

# partition choices: automatic, forced one pass, forced splits
PARTS = {1: [0, 16], 2: [0, 4096, 256], 3: [0, 8192, 512], 4: [0, 1024], 5: [0, 256]}


@functools.lru_cache(maxsize=1)
def _wl(cid):
    return workloads.build(cid)


def _fresh(wl, layer):
    dw = upload(wl, layers=[layer])
    d = dw.layers[0]
    poison_tails_gpu(wl, d)
    return dw, d


def _poison_slots(wl, dw, d, slots):
    nan = to_dev(workloads.nan_tokens(len(slots), wl.cfg), wl.cfg.dtype)
    pkv.kv_append(nan, nan, slots, d.k_cache, d.v_cache)


def _fused(wl, dw, d, pt=0, slots=None, lens=None, max_context_len=None):
    mcl = int(wl.context_lens.max()) if max_context_len is None else max_context_len
    return pkv.append_paged_attn_decode(d.q, d.k_new, d.v_new, dw.slots if slots is None else slots, d.k_cache,
                                        d.v_cache, dw.tables, dw.lens if lens is None else lens, wl.cfg.scale,
                                        max_context_len=max(mcl, 0), partition_tokens=pt)


def _two_calls(wl, dw, d, pt=0, slots=None, lens=None, max_context_len=None):
    pkv.kv_append(d.k_new, d.v_new, dw.slots if slots is None else slots, d.k_cache, d.v_cache)
    return gpu_decode(wl, dw, d, impl="mfma", partition_tokens=pt, lens=lens, max_context_len=max_context_len)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_fused_equals_append_then_decode(cid):
    wl = _wl(cid)
    layers = range(len(wl.layers)) if cid == 5 else [0]
    for li in layers:
        kc_ref, vc_ref = oracle_caches(wl, li)
        ref = oracle_decode(wl, li, kc_ref, vc_ref)
        for pt in PARTS[cid]:
            dwa, da = _fresh(wl, li)
            out_a = to_bits(_two_calls(wl, dwa, da, pt))
            ka, va = to_bits(da.k_cache).ravel(), to_bits(da.v_cache).ravel()
            del dwa, da
            dwb, db = _fresh(wl, li)
            _poison_slots(wl, dwb, db, dwb.slots)
            out_b = to_bits(_fused(wl, dwb, db, pt))
            kb, vb = to_bits(db.k_cache).ravel(), to_bits(db.v_cache).ravel()
            del dwb, db
            assert np.array_equal(kb, kc_ref) and np.array_equal(vb, vc_ref), f"layer {li} partition {pt}: pools"
            assert np.array_equal(ka, kb) and np.array_equal(va, vb)
            assert np.array_equal(out_a, out_b), f"layer {li} partition {pt}: output differs from two calls"
            r, e = assert_parity(out_b, ref, wl.cfg.dtype, f"config {cid} layer {li} partition {pt}")
            print(f"config {cid} layer {li} partition {pt}: fused == two calls, max|err| {e:.2e}", flush=True)


def _custom(lens, Hq=8, Hkv=2, D=64, bs=16, dtype="bf16", seed=11):
    wl = workloads.custom(Hq, Hkv, D, bs, lens, dtype, seed=seed, spare_blocks=2)
    return wl


@pytest.mark.parametrize("Hq,Hkv,D,bs,dtype", [(8, 2, 64, 512, "bf16"), (16, 2, 128, 1024, "fp16")])
def test_fused_large_block_sizes(Hq, Hkv, D, bs, dtype):
    """Fused == two calls, and within tolerance of the oracle, at block sizes 512 and
    1024; lengths across block edges, so the appended token lands at many offsets."""
    lens = [1, 512, 513, 1024, 1025, 2047, 2049, 3000]
    wl = _custom(lens, Hq=Hq, Hkv=Hkv, D=D, bs=bs, dtype=dtype, seed=bs)
    kc_ref, vc_ref = oracle_caches(wl, 0)
    ref = oracle_decode(wl, 0, kc_ref, vc_ref)
    for pt in (0, 512):
        dwa, da = _fresh(wl, 0)
        out_a = to_bits(_two_calls(wl, dwa, da, pt))
        dwb, db = _fresh(wl, 0)
        _poison_slots(wl, dwb, db, dwb.slots)
        out_b = to_bits(_fused(wl, dwb, db, pt))
        assert np.array_equal(to_bits(db.k_cache).ravel(), kc_ref) and np.array_equal(to_bits(db.v_cache).ravel(),
                                                                                         vc_ref), f"bs {bs}: pools"
        assert np.array_equal(out_a, out_b), f"bs {bs} partition {pt}: output differs from two calls"
        r, e = assert_parity(out_b, ref, dtype, f"bs {bs} partition {pt}")
        print(f"bs {bs} partition {pt}: fused == two calls, max|err| {e:.2e}", flush=True)


def test_fused_very_long_context():
    """Fused == two calls, and within tolerance of the oracle, with a 131,072-token
    context beside short ones (the automatic split: tens of partitions per row) and
    in the host dispatch order."""
    lens = [131072, 1, 17, 5000]
    wl = _custom(lens, Hq=32, Hkv=8, D=64, bs=16, dtype="bf16", seed=131)
    kc_ref, vc_ref = oracle_caches(wl, 0)
    ref = oracle_decode(wl, 0, kc_ref, vc_ref)
    order = torch.from_numpy(pkv.decode_schedule(lens)).cuda()
    dwa, da = _fresh(wl, 0)
    out_a = to_bits(_two_calls(wl, dwa, da))
    for seq_order in (None, order):
        dwb, db = _fresh(wl, 0)
        _poison_slots(wl, dwb, db, dwb.slots)
        out_b = to_bits(pkv.append_paged_attn_decode(db.q, db.k_new, db.v_new, dwb.slots, db.k_cache, db.v_cache,
                                                     dwb.tables, dwb.lens, wl.cfg.scale, max_context_len=131072,
                                                     seq_order=seq_order))
        assert np.array_equal(to_bits(db.k_cache).ravel(), kc_ref) and np.array_equal(to_bits(db.v_cache).ravel(),
                                                                                         vc_ref), "pools"
        assert np.array_equal(out_a, out_b), f"order {seq_order is not None}: output differs from two calls"
        r, e = assert_parity(out_b, ref, "bf16", "L 131072 fused")
        print(f"L 131072 fused (order {seq_order is not None}) == two calls, max|err| {e:.2e}", flush=True)


def test_fused_length_one_is_exactly_v_new():
    """With L = 1 the appended token is the whole context: out = v_new exactly."""
    wl = _custom([1] * 7, Hq=8, Hkv=2)
    dw, d = _fresh(wl, 0)
    _poison_slots(wl, dw, d, dw.slots)
    out = to_bits(_fused(wl, dw, d))
    vn = wl.layers[0].v_new
    for h in range(8):
        assert np.array_equal(out[:, h, :], vn[:, h // 4, :])


@pytest.mark.parametrize("pt", [0, 16])
def test_fused_wrong_and_missing_slots(pt):
    """A slot that is not the slot of position L-1: nothing written, that
    sequence's output NaN; a negative slot: nothing appended; the others as
    with the two calls."""
    lens = [5, 37, 16, 33, 40]
    wl = _custom(lens, Hq=4, Hkv=2)
    bs = wl.cfg.block_size
    slots = torch.from_numpy(wl.slot_mapping.copy())
    wrong = int(wl.block_tables[1, 1]) * bs + 3   # a position of sequence 1 other than L-1 = 36
    slots[1] = wrong
    slots[3] = -1
    # two-call reference: nothing appended for sequences 1 and 3
    ref_slots = slots.clone()
    ref_slots[1] = -1
    dwa, da = _fresh(wl, 0)
    out_a = to_bits(_two_calls(wl, dwa, da, pt, slots=ref_slots.cuda()))
    ka, va = to_bits(da.k_cache), to_bits(da.v_cache)
    dwb, db = _fresh(wl, 0)
    out_b = to_bits(_fused(wl, dwb, db, pt, slots=slots.cuda()))
    kb, vb = to_bits(db.k_cache), to_bits(db.v_cache)
    assert np.array_equal(ka, kb) and np.array_equal(va, vb), "pools differ: the wrong slot must not be written"
    got = bits_to_f64(out_b, "bf16")
    assert np.isnan(got[1]).all()
    for i in (0, 2, 3, 4):
        assert np.array_equal(out_a[i], out_b[i]), i


def test_fused_empty_context():
    """L = 0 without a slot: zeros; L = 0 with a slot: NaN and nothing written."""
    lens = [0, 5, 0, 20]
    wl = _custom(lens, Hq=4, Hkv=2)
    slots = torch.from_numpy(wl.slot_mapping.copy())
    assert slots[0] == -1 and slots[2] == -1
    slots[2] = int(wl.block_tables[1, 0]) * wl.cfg.block_size + 7  # any slot: L = 0 cannot take a token
    dw, d = _fresh(wl, 0)
    k0, v0 = to_bits(d.k_cache), to_bits(d.v_cache)
    out = bits_to_f64(to_bits(_fused(wl, dw, d, slots=slots.cuda())), "bf16")
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert np.isnan(out[2]).all()
    # only the slots of sequences 1 and 3 changed
    k1 = to_bits(d.k_cache)
    changed = np.unique(np.nonzero((k1 != k0).reshape(wl.num_blocks, -1))[0])
    assert set(changed.tolist()) <= {int(wl.block_tables[1, 0]), int(wl.block_tables[3, 1])}


def test_fused_checks_shapes():
    wl = _wl(1)
    dw, d = _fresh(wl, 0)
    with pytest.raises(pkv.PkvError):
        pkv.append_paged_attn_decode(d.q, d.k_new[:, :1], d.v_new, dw.slots, d.k_cache, d.v_cache, dw.tables,
                                     dw.lens, 0.125)

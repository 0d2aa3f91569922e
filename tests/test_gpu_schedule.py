"""Decode with a dispatch order (seq_order) on the GPU, through the C ABI.

The order only decides which workgroup decodes which sequence, so the outputs
(and, fused, the pools) must be bit-identical to the plain sequence order, for
the host schedule and for a random permutation, on the single-pass and split
plans, for the 16-bit, SIMT and FP8 kernels; and within tolerance of the oracle."""
import numpy as np
import pytest
import torch

import paged_kv_cache_448_amd as pkv
import workloads
from gpu_harness import assert_parity, oracle_caches, oracle_decode, poison_tails_gpu, to_bits, upload

pytestmark = pytest.mark.gpu


def _wl(cid):
    return workloads.build_config(workloads.CONFIGS[cid], seed=cid, num_layers=1)


def _orders(wl):
    B = len(wl.context_lens)
    rng = np.random.default_rng(7)
    return {"schedule": pkv.decode_schedule(wl.context_lens), "random": rng.permutation(B).astype(np.int32)}


def _fresh(wl):
    dw = upload(wl, layers=[0])
    poison_tails_gpu(wl, dw.layers[0])
    return dw, dw.layers[0]


@pytest.mark.parametrize("cid,impl,pt", [(1, "mfma", 0), (2, "mfma", 0), (2, "simt", 0), (2, "mfma", 256),
                                         (3, "mfma", 0), (4, "mfma", 0), (5, "mfma", 0)])
def test_decode_with_order_is_bit_identical(cid, impl, pt):
    wl = _wl(cid)
    c = wl.cfg
    mcl = int(wl.context_lens.max())
    dw, d = _fresh(wl)
    base = to_bits(pkv.paged_attn_decode(d.q, d.k_cache, d.v_cache, dw.tables, dw.lens, c.scale, max_context_len=mcl,
                                         partition_tokens=pt, impl=impl))
    for name, order in _orders(wl).items():
        out = pkv.paged_attn_decode(d.q, d.k_cache, d.v_cache, dw.tables, dw.lens, c.scale, max_context_len=mcl,
                                    partition_tokens=pt, impl=impl, seq_order=torch.from_numpy(order).cuda())
        assert np.array_equal(to_bits(out), base), f"config {cid} {impl} partition {pt}: {name} order differs"
    if cid in (2, 3) and impl == "mfma" and pt == 0:
        kc, vc = oracle_caches(wl, 0, append=False)
        assert_parity(base, oracle_decode(wl, 0, kc, vc), c.dtype, f"config {cid}")
    print(f"config {cid} {impl} partition {pt}: scheduled and random orders bit-identical", flush=True)


@pytest.mark.parametrize("cid", [2, 3, 5])
def test_fused_with_order_is_bit_identical(cid):
    wl = _wl(cid)
    c = wl.cfg
    mcl = int(wl.context_lens.max())
    results = []
    for order in (None, _orders(wl)["schedule"]):
        dw, d = _fresh(wl)
        so = None if order is None else torch.from_numpy(order).cuda()
        out = pkv.append_paged_attn_decode(d.q, d.k_new, d.v_new, dw.slots, d.k_cache, d.v_cache, dw.tables, dw.lens,
                                           c.scale, max_context_len=mcl, seq_order=so)
        results.append((to_bits(out), to_bits(d.k_cache), to_bits(d.v_cache)))
        del dw, d
    for a, b in zip(*results):
        assert np.array_equal(a, b), f"config {cid}: fused call with the schedule differs"
    kc, vc = oracle_caches(wl, 0)
    assert_parity(results[1][0], oracle_decode(wl, 0, kc, vc), c.dtype, f"config {cid} fused, scheduled")


def test_fp8_decode_with_order_is_bit_identical():
    wl = _wl(2)
    c = wl.cfg
    N, Hkv, bs, D = wl.num_blocks, c.num_kv_heads, c.block_size, c.head_dim
    dw, d = _fresh(wl)

    def rows(t):  # every slot of a 16-bit pool as [N*bs, Hkv, D]
        return t.permute(0, 2, 1, 3).reshape(N * bs, Hkv, D).contiguous()

    slots = torch.arange(N * bs, dtype=torch.int64, device="cuda")
    kp, vp = pkv.new_cache_fp8(N, Hkv, bs, D, "cuda"), pkv.new_cache_fp8(N, Hkv, bs, D, "cuda")
    pkv.kv_append_fp8(rows(d.k_cache), rows(d.v_cache), slots, kp, vp, 0.0125, 0.01)
    mcl = int(wl.context_lens.max())
    outs = []
    for order in (None, _orders(wl)["schedule"], _orders(wl)["random"]):
        so = None if order is None else torch.from_numpy(order).cuda()
        out = pkv.paged_attn_decode_fp8(d.q, kp, vp, dw.tables, dw.lens, c.scale, 0.0125, 0.01, max_context_len=mcl,
                                        seq_order=so)
        outs.append(to_bits(out))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_order_entries_outside_the_batch_are_skipped():
    """Slots whose entry is out of range decode nothing; the others are unchanged."""
    wl = _wl(2)
    c = wl.cfg
    mcl = int(wl.context_lens.max())
    dw, d = _fresh(wl)
    base = to_bits(pkv.paged_attn_decode(d.q, d.k_cache, d.v_cache, dw.tables, dw.lens, c.scale, max_context_len=mcl))
    order = np.arange(len(wl.context_lens), dtype=np.int32)
    order[[0, 5]] = [-1, 1 << 20]
    out = pkv.paged_attn_decode(d.q, d.k_cache, d.v_cache, dw.tables, dw.lens, c.scale, max_context_len=mcl,
                                seq_order=torch.from_numpy(order).cuda())
    keep = np.ones(len(order), bool)
    keep[[0, 5]] = False
    assert np.array_equal(to_bits(out)[keep], base[keep])

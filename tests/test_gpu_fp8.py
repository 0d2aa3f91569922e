"""FP8 (E4M3) KV cache on the GPU against the oracle (oracle.fp8): the quantising
append byte for byte (whole pools compared), and decode over FP8 pools within the
decode tolerance |gpu - oracle| <= 1e-2 + 1e-2 |oracle|.

Both sides start from the same generator arrays (16-bit token rows); each side
quantises them with its own append, and the pools are compared before the decode
is.  Every slot outside the contexts holds the NaN code, so tails and unused
blocks are poisoned as in the 16-bit tests.
"""
import functools
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_448_amd as pkv
import workloads
from gpu_harness import assert_parity, to_bits, to_dev
from oracle import fp8 as ofp8
from oracle.numerics import bits_to_f64

pytestmark = pytest.mark.gpu

# N(0,1) rows: |x| / scale reaches the top of the E4M3 range for the largest
# values (a few saturate), and small values land among the subnormals
K_SCALE, V_SCALE = 0.0125, 0.01

# inputs whose codes the format fixes at scale 1: signed zeros, saturation,
# infinities, NaN, ties to even, the subnormal boundaries
SPECIAL = [0.0, -0.0, math.inf, -math.inf, math.nan, 448.0, -448.0, 464.0, 480.0, 1.0e4, -1.0e4, 1.0625, 1.1875,
           -1.0625, 2.0 ** -10, 3 * 2.0 ** -11, 31 * 2.0 ** -11, 2.0 ** -9, 1.0e-6, 240.0, 0.5, -0.3]


def _special_bits(n, dtype, rng):
    x = np.concatenate([np.array(SPECIAL, dtype=np.float32), rng.standard_normal(n, dtype=np.float32) * 100])
    return workloads.f32_to_bits(x[:n], dtype)


@pytest.mark.parametrize("Hkv,D,bs,dtype,scales", [
    (8, 64, 16, "bf16", (K_SCALE, V_SCALE)), (4, 128, 256, "fp16", (K_SCALE, V_SCALE)),
    (1, 8, 32, "bf16", (1.0, 1.0)), (2, 64, 16, "fp16", (1.0, 1.0)), (2, 512, 1024, "bf16", (0.5, 3.0)),
])
def test_append_fp8_bit_exact(Hkv, D, bs, dtype, scales):
    """T tokens into distinct random slots, with padding tokens (-1) and slots beyond
    the pool (ignored); the first rows carry the special values."""
    rng = np.random.default_rng(D * 11 + bs)
    N = 37
    total = N * bs
    T = min(total, 900)
    slots = rng.permutation(total)[:T].astype(np.int64)
    slots[::17] = -1
    slots[5::23] = total + rng.integers(0, 1000, size=len(slots[5::23]))
    k = workloads.random_bits(rng, (T, Hkv, D), dtype)
    v = workloads.random_bits(rng, (T, Hkv, D), dtype)
    n_sp = min(T * Hkv * D, 4 * len(SPECIAL) + 64)
    k.reshape(-1)[:n_sp] = _special_bits(n_sp, dtype, rng)
    v.reshape(-1)[:n_sp] = _special_bits(n_sp, dtype, rng)[::-1]
    kc = rng.integers(0, 256, size=(N, Hkv, bs, D), dtype=np.uint8)
    vc = rng.integers(0, 256, size=(N, Hkv, bs, D), dtype=np.uint8)
    dk, dv = torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda()
    ks, vs = scales
    pkv.kv_append_fp8(to_dev(k, dtype), to_dev(v, dtype), torch.from_numpy(slots).cuda(), dk, dv, ks, vs)
    keep = slots < total
    ok, ov = kc.copy(), vc.copy()
    ofp8.append(k[keep], v[keep], dtype, slots[keep], ok, ov, ks, vs, num_blocks=N, block_size=bs)
    gk, gv = dk.cpu().numpy(), dv.cpu().numpy()
    assert np.array_equal(gk, ok), f"K pool: {np.count_nonzero(gk != ok)} bytes differ"
    assert np.array_equal(gv, ov), f"V pool: {np.count_nonzero(gv != ov)} bytes differ"


def _context_slots(wl):
    """Distinct slots of every context position of every sequence."""
    bs = wl.cfg.block_size
    out = []
    for i, L in enumerate(wl.context_lens):
        pos = np.arange(int(L), dtype=np.int64)
        out.append(wl.block_tables[i, pos // bs].astype(np.int64) * bs + pos % bs)
    return np.unique(np.concatenate(out)) if out else np.zeros(0, np.int64)


@functools.lru_cache(maxsize=2)
def _prepared(key):
    """Workload, context slots, the 16-bit rows stored there, and the oracle's FP8 pools."""
    wl = _WORKLOADS[key]()
    c = wl.cfg
    N, Hkv, bs, D = wl.num_blocks, c.num_kv_heads, c.block_size, c.head_dim
    slots = _context_slots(wl)
    ly = wl.layers[0]

    def rows(pool):
        return np.ascontiguousarray(pool.reshape(N, Hkv, bs, D).transpose(0, 2, 1, 3).reshape(N * bs, Hkv, D)[slots])

    k_rows, v_rows = rows(ly.k_cache), rows(ly.v_cache)
    kc = np.full((N, Hkv, bs, D), ofp8.NAN_CODE, dtype=np.uint8)
    vc = np.full_like(kc, ofp8.NAN_CODE)
    ofp8.append(k_rows, v_rows, c.dtype, slots, kc, vc, K_SCALE, V_SCALE, num_blocks=N, block_size=bs)
    return wl, slots, k_rows, v_rows, kc, vc


@functools.lru_cache(maxsize=4)
def _reference(key):
    wl, _, _, _, kc, vc = _prepared(key)
    c = wl.cfg
    return ofp8.decode(wl.layers[0].q, kc, vc, K_SCALE, V_SCALE, wl.block_tables, wl.context_lens, c.scale,
                       q_dtype=c.dtype, num_blocks=wl.num_blocks, num_kv_heads=c.num_kv_heads, block_size=c.block_size)


_WORKLOADS = {
    "tiny": lambda: workloads.build(1),
    "llama3.2-1b-b64": lambda: workloads.build(2),
    "fp16-d128-g8-ragged": lambda: workloads.custom(16, 2, 128, 16, [1, 15, 16, 17, 700, 2100, 0, 333], "fp16",
                                                    seed=4),
    "fp16-d128-mha": lambda: workloads.custom(8, 8, 128, 32, [40, 1000, 257], "fp16", seed=5),
    "bf16-g16-bs256": lambda: workloads.custom(16, 1, 64, 256, [5000, 31, 2600], "bf16", seed=6),
    "bf16-bs512": lambda: workloads.custom(8, 2, 64, 512, [1, 511, 513, 1025, 2049], "bf16", seed=7),
    "fp16-d128-bs1024": lambda: workloads.custom(16, 2, 128, 1024, [17, 1023, 1025, 3000], "fp16", seed=8),
    # a 64k-token context beside short ones: tens of partitions per row for the merge
    "bf16-long-64k": lambda: workloads.custom(32, 8, 64, 16, [65536, 1, 17, 5000], "bf16", seed=9),
}
PARTS = {"tiny": [0, 16, 32], "llama3.2-1b-b64": [0, 4096, 128, 512], "fp16-d128-g8-ragged": [0, 2112, 256, 512],
         "fp16-d128-mha": [0, 128], "bf16-g16-bs256": [0, 8192, 256, 1024], "bf16-bs512": [0, 512, 1024],
         "fp16-d128-bs1024": [0, 1024, 256], "bf16-long-64k": [0, 8192]}


def _device_pools(key):
    wl, slots, k_rows, v_rows, _, _ = _prepared(key)
    c = wl.cfg
    shape = (wl.num_blocks, c.num_kv_heads, c.block_size, c.head_dim)
    kc = torch.full(shape, ofp8.NAN_CODE, dtype=torch.uint8, device="cuda")
    vc = torch.full(shape, ofp8.NAN_CODE, dtype=torch.uint8, device="cuda")
    pkv.kv_append_fp8(to_dev(k_rows, c.dtype), to_dev(v_rows, c.dtype), torch.from_numpy(slots).cuda(), kc, vc,
                      K_SCALE, V_SCALE)
    return kc, vc


@pytest.mark.parametrize("key", list(_WORKLOADS))
def test_decode_fp8_parity(key):
    wl, _, _, _, okc, ovc = _prepared(key)
    c = wl.cfg
    kc, vc = _device_pools(key)
    assert np.array_equal(kc.cpu().numpy(), okc), f"{key}: K pool differs from the oracle's append"
    assert np.array_equal(vc.cpu().numpy(), ovc), f"{key}: V pool differs from the oracle's append"
    ref = _reference(key)
    q = to_dev(wl.layers[0].q, c.dtype)
    tables = torch.from_numpy(wl.block_tables).cuda()
    lens = torch.from_numpy(wl.context_lens).cuda()
    mcl = max(int(wl.context_lens.max()), 0)
    for pt in PARTS[key]:
        out = pkv.paged_attn_decode_fp8(q, kc, vc, tables, lens, c.scale, K_SCALE, V_SCALE, max_context_len=mcl,
                                        partition_tokens=pt)
        r, e = assert_parity(to_bits(out), ref, c.dtype, f"{key} partition {pt}")
        print(f"{key} partition {pt}: max|err| {e:.2e} (ratio {r:.3f})", flush=True)
        empty = wl.context_lens == 0
        if empty.any():
            assert not to_bits(out)[empty].any(), "an empty sequence must give zeros"


def test_decode_fp8_invalid_inputs_give_nan_only_where_they_are():
    """A length above max_context_len and a block id outside the pool: NaN in those
    sequences' heads, the others still match the oracle."""
    key = "tiny"
    wl, _, _, _, _, _ = _prepared(key)
    c = wl.cfg
    kc, vc = _device_pools(key)
    ref = _reference(key)
    q = to_dev(wl.layers[0].q, c.dtype)
    mcl = int(wl.context_lens.max())
    lens = wl.context_lens.copy()
    lens[0] = mcl + 1
    out = pkv.paged_attn_decode_fp8(q, kc, vc, torch.from_numpy(wl.block_tables).cuda(), torch.from_numpy(lens).cuda(),
                                    c.scale, K_SCALE, V_SCALE, max_context_len=mcl)
    got = to_bits(out)
    assert np.all(np.isnan(bits_to_f64(got[0], c.dtype)))
    assert_parity(got[1:], ref[1:], c.dtype, "valid sequence next to an invalid length")
    tables = wl.block_tables.copy()
    tables[1, 1] = wl.num_blocks  # second block of sequence 1 is outside the pool
    out = pkv.paged_attn_decode_fp8(q, kc, vc, torch.from_numpy(tables).cuda(), torch.from_numpy(wl.context_lens).cuda(),
                                    c.scale, K_SCALE, V_SCALE, max_context_len=mcl)
    got = to_bits(out)
    assert np.all(np.isnan(bits_to_f64(got[1], c.dtype)))
    assert_parity(got[:1], ref[:1], c.dtype, "valid sequence next to a bad block id")


def test_fp8_rejects_bad_scales_and_dtypes():
    kc = pkv.new_cache_fp8(4, 2, 16, 64)
    k = torch.zeros((1, 2, 64), dtype=torch.bfloat16, device="cuda")
    slots = torch.zeros(1, dtype=torch.int64, device="cuda")
    for bad in (0.0, -1.0, math.inf, math.nan):
        with pytest.raises(pkv.PkvError):
            pkv.kv_append_fp8(k, k, slots, kc, kc.clone(), bad, 1.0)
    with pytest.raises(pkv.PkvError):
        pkv.kv_append_fp8(k, k, slots, kc.view(torch.int8), kc.clone(), 1.0, 1.0)
    q = torch.zeros((1, 4, 64), dtype=torch.float32, device="cuda")
    t = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PkvError):
        pkv.paged_attn_decode_fp8(q, kc, kc.clone(), t, t[0].clone(), 0.125, 1.0, 1.0)


FUSED_PARTS = {"tiny": [0, 16], "llama3.2-1b-b64": [0, 512], "fp16-d128-g8-ragged": [0, 256],
               "bf16-g16-bs256": [0, 1024], "bf16-bs512": [0, 512], "fp16-d128-bs1024": [0, 1024],
               "bf16-long-64k": [0]}


def _poisoned_fused_pools(key, slots):
    """The context pools with the append slots set to the NaN code, so that a read of
    a slot's old contents instead of the appended token would show."""
    wl = _prepared(key)[0]
    c = wl.cfg
    kc, vc = _device_pools(key)
    keep = slots[slots >= 0]
    if len(keep):
        nan = to_dev(workloads.nan_tokens(len(keep), c), c.dtype)
        pkv.kv_append_fp8(nan, nan, torch.from_numpy(keep).cuda(), kc, vc, K_SCALE, V_SCALE)
    return kc, vc


@pytest.mark.parametrize("key", list(FUSED_PARTS))
def test_fused_fp8_append_decode_equals_two_calls(key):
    """append_paged_attn_decode_fp8 against kv_append_fp8 + paged_attn_decode_fp8:
    pools byte-identical and outputs bit-identical; and within tolerance of the oracle
    over the oracle's own append."""
    wl, _, _, _, okc, ovc = _prepared(key)
    c = wl.cfg
    ly = wl.layers[0]
    q, kn, vn = to_dev(ly.q, c.dtype), to_dev(ly.k_new, c.dtype), to_dev(ly.v_new, c.dtype)
    slots = torch.from_numpy(wl.slot_mapping).cuda()
    tables = torch.from_numpy(wl.block_tables).cuda()
    lens = torch.from_numpy(wl.context_lens).cuda()
    mcl = max(int(wl.context_lens.max()), 0)
    okc, ovc = okc.copy(), ovc.copy()
    keep = wl.slot_mapping >= 0
    ofp8.append(ly.k_new[keep], ly.v_new[keep], c.dtype, wl.slot_mapping[keep], okc, ovc, K_SCALE, V_SCALE,
                num_blocks=wl.num_blocks, block_size=c.block_size)
    ref = ofp8.decode(ly.q, okc, ovc, K_SCALE, V_SCALE, wl.block_tables, wl.context_lens, c.scale, q_dtype=c.dtype,
                      num_blocks=wl.num_blocks, num_kv_heads=c.num_kv_heads, block_size=c.block_size)
    for pt in FUSED_PARTS[key]:
        ka, va = _device_pools(key)
        pkv.kv_append_fp8(kn, vn, slots, ka, va, K_SCALE, V_SCALE)
        out_a = to_bits(pkv.paged_attn_decode_fp8(q, ka, va, tables, lens, c.scale, K_SCALE, V_SCALE,
                                                  max_context_len=mcl, partition_tokens=pt))
        kb, vb = _poisoned_fused_pools(key, wl.slot_mapping)
        out_b = to_bits(pkv.append_paged_attn_decode_fp8(q, kn, vn, slots, kb, vb, tables, lens, c.scale, K_SCALE,
                                                         V_SCALE, max_context_len=mcl, partition_tokens=pt))
        assert np.array_equal(kb.cpu().numpy(), okc) and np.array_equal(vb.cpu().numpy(), ovc), \
            f"{key} partition {pt}: pools differ from the oracle's append"
        assert np.array_equal(ka.cpu().numpy(), kb.cpu().numpy()) and np.array_equal(va.cpu().numpy(),
                                                                                      vb.cpu().numpy())
        assert np.array_equal(out_a, out_b), f"{key} partition {pt}: fused output differs from two calls"
        r, e = assert_parity(out_b, ref, c.dtype, f"{key} fused partition {pt}")
        print(f"{key} partition {pt}: fused == two calls, max|err| {e:.2e}", flush=True)


def test_fused_fp8_wrong_and_missing_slots():
    """A slot that is not the slot of L-1 writes nothing and gives NaN in that
    sequence only; a negative slot appends nothing and decodes the pool as it is."""
    key = "llama3.2-1b-b64"
    wl = _prepared(key)[0]
    c = wl.cfg
    ly = wl.layers[0]
    q, kn, vn = to_dev(ly.q, c.dtype), to_dev(ly.k_new, c.dtype), to_dev(ly.v_new, c.dtype)
    tables = torch.from_numpy(wl.block_tables).cuda()
    lens = torch.from_numpy(wl.context_lens).cuda()
    mcl = int(wl.context_lens.max())
    slots = wl.slot_mapping.copy()
    # a sequence whose position L-2 shares the block of L-1: its slot is slot - 1,
    # inside its own context and no other sequence's append slot
    i = next(j for j in range(len(slots)) if (int(wl.context_lens[j]) - 1) % c.block_size != 0 and j != 7)
    wrong = int(slots[i] - 1)
    slots[i] = wrong
    slots[7] = -1
    kb, vb = _device_pools(key)
    before_k = kb.cpu().numpy().copy()
    out = to_bits(pkv.append_paged_attn_decode_fp8(q, kn, vn, torch.from_numpy(slots).cuda(), kb, vb, tables, lens,
                                                   c.scale, K_SCALE, V_SCALE, max_context_len=mcl))
    got = bits_to_f64(out, c.dtype)
    assert np.all(np.isnan(got[i])), "a wrong slot must make its sequence NaN"
    assert np.all(np.isfinite(np.delete(got, i, axis=0)))
    N, Hkv, bs, D = kb.shape
    after = kb.cpu().numpy().transpose(0, 2, 1, 3).reshape(N * bs, Hkv, D)
    assert np.array_equal(after[wrong], before_k.transpose(0, 2, 1, 3).reshape(N * bs, Hkv, D)[wrong])
    # sequence 7 (no append) decodes the pool's old row at L-1: same as the plain decode
    plain = to_bits(pkv.paged_attn_decode_fp8(q, kb, vb, tables, lens, c.scale, K_SCALE, V_SCALE,
                                              max_context_len=mcl))
    assert np.array_equal(out[7], plain[7])

"""Pins of the decode oracle against facts that do not come from the oracle itself.

Each pin takes a decode function with the signature of ``oracle.decode`` so the
mutant tests can rerun every pin on a deliberately broken copy.  Cases are built
by writing known logical K/V tokens into a shuffled pool through the oracle's
append (whose layout is stated as an offset formula, independently of the
array view the decode oracle reads through), so expected values come from
closed forms over the known tokens, from a library routine, or from the scalar
brute-force loops -- never from the function under test.
"""
import dataclasses
import math

import numpy as np

import oracle
import workloads
from oracle.numerics import bits_to_f64


@dataclasses.dataclass
class Case:
    wl: workloads.Workload
    q: np.ndarray          # uint16 [B, Hq, D]
    k_cache: np.ndarray
    v_cache: np.ndarray
    ctx_k: list            # per seq uint16 [L, Hkv, D] (logical order)
    ctx_v: list

    @property
    def cfg(self):
        return self.wl.cfg


def int_bits(a, dtype="bf16"):
    """Small integers (exact in bf16/fp16) as storage bits."""
    return workloads.f32_to_bits(np.asarray(a, dtype=np.float32), dtype)


def context_slots(wl, i):
    bs = wl.cfg.block_size
    t = np.arange(int(wl.context_lens[i]))
    return wl.block_tables[i, t // bs].astype(np.int64) * bs + t % bs


def make_case(Hq, Hkv, D, bs, lens, dtype="bf16", seed=0, ctx_k=None, ctx_v=None, q=None,
              spare_blocks=2):
    wl = workloads.custom(Hq, Hkv, D, bs, lens, dtype, seed=seed, spare_blocks=spare_blocks, poison=True)
    layer = wl.layers[0]
    rng = np.random.default_rng(seed + 7919)
    kc, vc = layer.k_cache.copy(), layer.v_cache.copy()
    N = wl.num_blocks
    if len(wl.tail_slots):
        nan = workloads.nan_tokens(len(wl.tail_slots), wl.cfg)
        oracle.kv_append(nan, nan, wl.tail_slots, kc, vc, num_blocks=N, block_size=bs)
    ks, vs = [], []
    for i, L in enumerate(lens):
        k = ctx_k[i] if ctx_k is not None else workloads.random_bits(rng, (L, Hkv, D), dtype)
        v = ctx_v[i] if ctx_v is not None else workloads.random_bits(rng, (L, Hkv, D), dtype)
        if L:
            oracle.kv_append(k, v, context_slots(wl, i), kc, vc, num_blocks=N, block_size=bs)
        ks.append(k)
        vs.append(v)
    qq = layer.q if q is None else q
    return Case(wl, qq, kc, vc, ks, vs)


def run(dec, case, scale=None, q=None, tables=None, k_cache=None, v_cache=None, num_blocks=None):
    c = case.cfg
    return dec(case.q if q is None else q,
               case.k_cache if k_cache is None else k_cache,
               case.v_cache if v_cache is None else v_cache,
               case.wl.block_tables if tables is None else tables,
               case.wl.context_lens, c.scale if scale is None else scale,
               dtype=c.dtype, num_blocks=case.wl.num_blocks if num_blocks is None else num_blocks,
               num_kv_heads=c.num_kv_heads, block_size=c.block_size)


def close(a, b, tol=1e-12):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.all(np.isfinite(a)), "non-finite output"
    err = np.abs(a - b) / (1.0 + np.abs(b))
    assert err.max() <= tol, f"max rel err {err.max():.3e} > {tol:.0e}"


# ---------------------------------------------------------------------------- pins

def pin_length_one_is_v0(dec):
    """With one context token the softmax weight is exactly 1: out = V_0 exactly."""
    case = make_case(8, 2, 16, 16, [1, 1, 1], seed=11)
    out = run(dec, case)
    G = 4
    for i in range(3):
        v0 = bits_to_f64(case.ctx_v[i][0], "bf16")   # [Hkv, D]
        for h in range(8):
            assert np.array_equal(out[i, h], v0[h // G]), "L=1 output is not V_0"


def pin_identical_keys_give_mean_v(dec):
    """All keys equal: uniform weights, out = mean of V over the context."""
    lens = [5, 37, 16]
    rng = np.random.default_rng(3)
    ks = [np.broadcast_to(workloads.random_bits(rng, (1, 2, 16), "bf16"), (L, 2, 16)).copy() for L in lens]
    case = make_case(4, 2, 16, 16, lens, seed=12, ctx_k=ks)
    out = run(dec, case)
    for i, L in enumerate(lens):
        mv = bits_to_f64(case.ctx_v[i], "bf16").mean(axis=0)    # [Hkv, D]
        close(out[i], mv[np.arange(4) // 2])


def pin_scale_zero_gives_mean_v(dec):
    case = make_case(4, 1, 16, 32, [45, 3], seed=13)
    out = run(dec, case, scale=0.0)
    for i in range(2):
        mv = bits_to_f64(case.ctx_v[i], "bf16").mean(axis=0)
        close(out[i], np.repeat(mv, 4, axis=0))


def pin_key_shift_invariance(dec):
    """q.(k+u) = q.k + q.u, constant over tokens: the softmax does not move."""
    lens = [21, 40]
    rng = np.random.default_rng(4)
    kint = [rng.integers(-4, 5, size=(L, 2, 8)) for L in lens]
    u = rng.integers(-4, 5, size=(1, 2, 8))
    qint = rng.integers(-3, 4, size=(2, 4, 8))
    q = int_bits(qint)
    base = make_case(4, 2, 8, 16, lens, seed=14, ctx_k=[int_bits(k) for k in kint], q=q)
    shifted = make_case(4, 2, 8, 16, lens, seed=14, ctx_k=[int_bits(k + u) for k in kint],
                        ctx_v=base.ctx_v, q=q)
    close(run(dec, shifted), run(dec, base))


def pin_linear_in_v(dec):
    lens = [17, 33]
    rng = np.random.default_rng(5)
    v1 = [rng.integers(-8, 9, size=(L, 2, 16)) for L in lens]
    v2 = [rng.integers(-8, 9, size=(L, 2, 16)) for L in lens]
    c1 = make_case(4, 2, 16, 16, lens, seed=15, ctx_v=[int_bits(v) for v in v1])
    c2 = make_case(4, 2, 16, 16, lens, seed=15, ctx_k=c1.ctx_k, ctx_v=[int_bits(v) for v in v2], q=c1.q)
    c3 = make_case(4, 2, 16, 16, lens, seed=15, ctx_k=c1.ctx_k,
                   ctx_v=[int_bits(a + 2 * b) for a, b in zip(v1, v2)], q=c1.q)
    close(run(dec, c3), run(dec, c1) + 2 * run(dec, c2))


def pin_dominant_key(dec):
    """One key whose score beats every other by >= 50 takes all the weight."""
    lens = [30]
    rng = np.random.default_rng(6)
    k = rng.integers(-2, 3, size=(30, 1, 8))
    k[17, 0, :] = 64            # its score is about 1448; every other one is at most about 45
    q = int_bits(np.full((1, 2, 8), 8))
    case = make_case(2, 1, 8, 16, lens, seed=16, ctx_k=[int_bits(k)], q=q)
    s = case.cfg.scale * 8 * k[:, 0, :].sum(axis=1)
    assert np.sort(s)[-1] - np.sort(s)[-2] >= 50
    out = run(dec, case)
    close(out[0], np.repeat(bits_to_f64(case.ctx_v[0][17], "bf16"), 2, axis=0))


def pin_gqa_grouping(dec):
    """kv head g holds V = g everywhere: q head h must output h // G."""
    lens = [9, 26]
    Hq, Hkv = 8, 4
    vs = [int_bits(np.broadcast_to(np.arange(Hkv)[None, :, None], (L, Hkv, 16))) for L in lens]
    case = make_case(Hq, Hkv, 16, 16, lens, seed=17, ctx_v=vs)
    out = run(dec, case)
    want = np.broadcast_to((np.arange(Hq) // (Hq // Hkv))[None, :, None].astype(np.float64), out.shape)
    close(out, want)


def pin_block_permutation_invariance(dec):
    """Moving physical blocks (and their table entries) changes nothing, bit for bit."""
    case = make_case(4, 2, 16, 16, [5, 37, 50], seed=18, spare_blocks=3)
    wl = case.wl
    N, E = wl.num_blocks, wl.block_elems
    perm = np.random.default_rng(8).permutation(N)
    kc = np.empty_like(case.k_cache)
    vc = np.empty_like(case.v_cache)
    for n in range(N):
        kc[perm[n] * E:(perm[n] + 1) * E] = case.k_cache[n * E:(n + 1) * E]
        vc[perm[n] * E:(perm[n] + 1) * E] = case.v_cache[n * E:(n + 1) * E]
    tables = perm[wl.block_tables].astype(np.int32)
    a = run(dec, case)
    b = run(dec, case, tables=tables, k_cache=kc, v_cache=vc)
    assert np.array_equal(a, b)


def pin_nan_poison_unreached(dec):
    """Tail slots, unused blocks and table padding hold NaN; the output stays finite."""
    case = make_case(4, 2, 16, 16, [1, 15, 16, 17, 40], seed=19)
    assert np.isnan(bits_to_f64(case.k_cache, "bf16")).any()
    out = run(dec, case)
    assert np.all(np.isfinite(out))


def pin_empty_context_is_zero(dec):
    case = make_case(4, 2, 16, 16, [0, 7], seed=20)
    out = run(dec, case)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert np.all(np.isfinite(out[1]))


def pin_brute_force(dec, trials=12):
    """Agreement with the scalar-loop reference on random tiny shapes."""
    rng = np.random.default_rng(21)
    for trial in range(trials):
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 3]))
        D = int(rng.choice([8, 16]))
        bs = int(rng.choice([16, 32]))
        lens = [int(x) for x in rng.integers(1, 41, size=int(rng.integers(1, 4)))]
        dtype = "bf16" if trial % 3 else "fp16"
        case = make_case(G * Hkv, Hkv, D, bs, lens, dtype=dtype, seed=100 + trial)
        c = case.cfg
        ref = oracle.brute.decode(case.q, case.k_cache, case.v_cache, case.wl.block_tables,
                                  case.wl.context_lens, c.scale, dtype=dtype, num_kv_heads=Hkv,
                                  block_size=bs)
        close(run(dec, case), ref)


def pin_library_sdpa(dec):
    """Agreement with torch's scaled_dot_product_attention (float64, its own GQA
    convention) on the logical contexts, for bf16 and fp16."""
    import torch
    import torch.nn.functional as F
    for dtype, (Hq, Hkv, D, bs, lens) in (("bf16", (8, 2, 64, 16, [5, 37, 64, 100])),
                                           ("fp16", (4, 4, 128, 16, [33, 16])),
                                           ("bf16", (8, 4, 64, 256, [300, 257]))):
        case = make_case(Hq, Hkv, D, bs, lens, dtype=dtype, seed=22)
        out = run(dec, case)
        qf = bits_to_f64(case.q, dtype)
        for i, L in enumerate(lens):
            k = torch.from_numpy(bits_to_f64(case.ctx_k[i], dtype)).permute(1, 0, 2)[None]  # [1,Hkv,L,D]
            v = torch.from_numpy(bits_to_f64(case.ctx_v[i], dtype)).permute(1, 0, 2)[None]
            qq = torch.from_numpy(qf[i])[None, :, None, :]                                # [1,Hq,1,D]
            ref = F.scaled_dot_product_attention(qq, k, v, scale=case.cfg.scale, enable_gqa=True)
            close(out[i], ref[0, :, 0, :].numpy())


ALL_PINS = [pin_length_one_is_v0, pin_identical_keys_give_mean_v, pin_scale_zero_gives_mean_v,
            pin_key_shift_invariance, pin_linear_in_v, pin_dominant_key, pin_gqa_grouping,
            pin_block_permutation_invariance, pin_nan_poison_unreached, pin_empty_context_is_zero,
            pin_brute_force, pin_library_sdpa]

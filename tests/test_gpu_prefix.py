"""paged_attn_decode_prefix on the GPU: shared prefixes read once per prefix
item, against the fp64 oracle (which reads every sequence's own blocks).

Tolerance as every decode test: |gpu - oracle| <= 1e-2 + 1e-2 |oracle|
elementwise, no NaN/Inf.  Fused calls also leave the pools bit-identical to
the oracle's append.  Cases: the 16-layer continuous-batching step (shared
512-token prompt prefix, 8 groups of 32), every GQA group size and both head
dims, lengths around block edges, forced partitions, prefixes longer than one
prefix chunk, a dispatch order, and plans that lie about the sharing (those
sequences must come out NaN, the others unchanged).
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


@functools.lru_cache(maxsize=1)
def _wl5():
    return workloads.build(5)


def _shared(Hq, Hkv, D, bs, lens, groups, prefix_blocks, dtype="bf16", seed=0):
    cfg = workloads.Config(0, "custom-shared", 1, len(lens), Hq, Hkv, D, bs, dtype, "fixed",
                           fixed_lens=tuple(int(x) for x in lens), prefix_groups=groups, prefix_blocks=prefix_blocks)
    return workloads.build_config(cfg, seed=seed)


def _plan(wl):
    c = wl.cfg
    return pkv.decode_prefix_plan(wl.block_tables, wl.context_lens, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                  c.block_size)


def _dev_plan(plan):
    items = plan.items if plan.num_items else np.full((1, 16), -1, np.int32)
    return torch.from_numpy(plan.prefix_len).cuda(), torch.from_numpy(np.ascontiguousarray(items)).cuda()


def _run(wl, layer, plan, fused, pt=0, prefix_len=None, seq_order=None, num_items=None, work=None):
    """One prefix decode of `layer` on fresh device pools; returns (out bits, k pool bits, v pool bits)."""
    c = wl.cfg
    dw = upload(wl, layers=[layer])
    d = dw.layers[0]
    poison_tails_gpu(wl, d)
    pl, items = _dev_plan(plan)
    if prefix_len is not None:
        pl = torch.from_numpy(np.asarray(prefix_len, dtype=np.int32)).cuda()
    if num_items is not None:
        items = items[:num_items]
    if fused:
        # the slots hold NaN before the fused call: a read of the old contents would show
        nan = to_dev(workloads.nan_tokens(len(wl.slot_mapping), c), c.dtype)
        pkv.kv_append(nan, nan, dw.slots, d.k_cache, d.v_cache)
        kw = dict(k_new=d.k_new, v_new=d.v_new, slot_mapping=dw.slots)
    else:
        pkv.kv_append(d.k_new, d.v_new, dw.slots, d.k_cache, d.v_cache)
        kw = {}
    out = pkv.paged_attn_decode_prefix(d.q, d.k_cache, d.v_cache, dw.tables, dw.lens, c.scale, pl, items,
                                       plan.max_prefix_len, max_context_len=max(int(wl.context_lens.max()), 0),
                                       partition_tokens=pt, seq_order=seq_order,
                                       work=None if work is None else torch.from_numpy(work).cuda(), **kw)
    res = to_bits(out), to_bits(d.k_cache).ravel(), to_bits(d.v_cache).ravel()
    del dw, d
    return res


def _check(wl, layer, plan, fused, pt=0, what="", ref=None, caches=None):
    kc, vc = oracle_caches(wl, layer) if caches is None else caches
    if ref is None:
        ref = oracle_decode(wl, layer, kc, vc)
    out, kg, vg = _run(wl, layer, plan, fused, pt)
    if fused:
        assert np.array_equal(kg, kc) and np.array_equal(vg, vc), f"{what}: pools differ from the oracle's append"
    r, e = assert_parity(out, ref, wl.cfg.dtype, what)
    print(f"{what}: items {plan.num_items}, longest prefix {plan.max_prefix_len}, max|err| {e:.2e} "
          f"(ratio {r:.3f})", flush=True)
    return out


def test_cb_step_all_layers_fused():
    """All 16 layers of the continuous-batching step, append fused, automatic plan."""
    wl = _wl5()
    plan = _plan(wl)
    assert plan.num_items > 0 and plan.max_prefix_len == 512
    for li in range(len(wl.layers)):
        _check(wl, li, plan, True, what=f"config 5 layer {li} fused")


@pytest.mark.parametrize("pt", [256, 1536, 8192])
def test_cb_step_partitions(pt):
    wl = _wl5()
    plan = _plan(wl)
    for li in (0, 9):
        _check(wl, li, plan, pt != 1536, pt, what=f"config 5 layer {li} partition {pt}")


def test_cb_step_order_and_determinism():
    """A dispatch order changes only which workgroup takes which sequence:
    bit-identical outputs; and two runs are bit-identical."""
    wl = _wl5()
    plan = _plan(wl)
    order = torch.from_numpy(pkv.decode_schedule(wl.context_lens)).cuda()
    a = _run(wl, 3, plan, True)[0]
    b = _run(wl, 3, plan, True)[0]
    c = _run(wl, 3, plan, True, seq_order=order)[0]
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_cb_step_matches_plain_decode():
    """Against the plain decode of the same inputs: equal up to the rounding of
    P to bf16 against a running maximum that depends on the work split (the
    bound of the decode tests' plan-agreement check: 8u absolute)."""
    wl = _wl5()
    plan = _plan(wl)
    dw = upload(wl, layers=[5])
    d = dw.layers[0]
    poison_tails_gpu(wl, d)
    pkv.kv_append(d.k_new, d.v_new, dw.slots, d.k_cache, d.v_cache)
    plain = to_bits(gpu_decode(wl, dw, d, impl="mfma"))
    del dw, d
    pre = _run(wl, 5, plan, False)[0]
    a, b = bits_to_f64(pre, "bf16"), bits_to_f64(plain, "bf16")
    ratio = float((np.abs(a - b) / (8 * 2.0 ** -9 + 2.0 ** -7 * np.abs(b))).max())
    print(f"prefix vs plain decode: ratio to bound {ratio:.3f}", flush=True)
    assert ratio <= 1.0


SHAPES = [
    # Hq, Hkv, D, bs, dtype, groups, prefix blocks
    (32, 8, 64, 16, "bf16", 4, 6),
    (16, 16, 128, 16, "fp16", 2, 9),      # G = 1: 16 members per item
    (64, 4, 64, 32, "bf16", 4, 5),        # G = 16: 2 members per item
    (8, 4, 128, 64, "fp16", 4, 3),        # G = 2 at head_dim 128: 8 members
    (16, 2, 64, 256, "bf16", 2, 2),       # G = 8, large blocks
    (16, 8, 64, 1024, "fp16", 2, 2),      # G = 2, the largest block size
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}q{s[1]}kv-d{s[2]}-bs{s[3]}-{s[4]}")
def test_shapes_block_edges_partitions(shape):
    Hq, Hkv, D, bs, dt, groups, pb = shape
    edges = [0, 1, 2, 17, bs, bs + 1, 2 * bs, 2 * bs + 1, 3 * bs + 1, pb * bs, pb * bs + 1, pb * bs + 2,
             (pb + 1) * bs + 1, (pb + 3) * bs + 5]
    per_group = len(edges)
    lens = np.array([e for _ in range(groups) for e in edges])
    wl = _shared(Hq, Hkv, D, bs, lens, groups, pb, dt, seed=3)
    plan = _plan(wl)
    assert plan.num_items > 0 or Hq // Hkv == 16 and D == 128
    kc, vc = oracle_caches(wl, 0)
    ref = oracle_decode(wl, 0, kc, vc)
    for pt in (0, 16, 48, bs * 2):
        for fused in (False, True):
            _check(wl, 0, plan, fused, pt, what=f"{shape} partition {pt} fused {fused}", ref=ref, caches=(kc, vc))
    assert per_group * groups == len(lens)


def test_long_prefixes_several_chunks():
    """Prefixes of up to 2400 tokens: 1024-token prefix chunks, up to three per member."""
    bs, pb = 16, 150
    lens = np.array([2400 + 1, 2400 + 2, 3000, 2400 + 16, 1000, 2401, 4000, 33, 1600, 2500, 2417, 2402] * 2)
    wl = _shared(32, 8, 64, bs, lens, 2, pb, "bf16", seed=5)
    plan = _plan(wl)
    assert plan.max_prefix_len == 2400
    kc, vc = oracle_caches(wl, 0)
    ref = oracle_decode(wl, 0, kc, vc)
    for pt in (0, 512):
        _check(wl, 0, plan, True, pt, what=f"long prefixes partition {pt}", ref=ref, caches=(kc, vc))


def test_empty_plan_is_plain_decode():
    """No items: the call is the plain MFMA decode, bit for bit."""
    wl = workloads.custom(32, 8, 64, 16, [5, 100, 2000, 0, 1, 700], "bf16", seed=1)
    plan = _plan(wl)
    assert plan.num_items == 0
    dw = upload(wl, layers=[0])
    d = dw.layers[0]
    poison_tails_gpu(wl, d)
    pkv.kv_append(d.k_new, d.v_new, dw.slots, d.k_cache, d.v_cache)
    plain = to_bits(gpu_decode(wl, dw, d, impl="mfma"))
    del dw, d
    assert np.array_equal(_run(wl, 0, plan, False)[0], plain)


def _expected_nan(pl, lens, items, tables, bs, max_pl):
    """Sequences the kernel must turn into NaN for a prefix plan (its stated
    rules): an unusable length (not 0 or a multiple of 16 below L, or above the
    bound); or a member whose reference is unusable, whose length exceeds the
    reference's, or whose table differs from the reference's within it."""
    ok = lambda s: pl[s] == 0 or (pl[s] % 16 == 0 and 0 < pl[s] <= lens[s] - 1 and pl[s] <= max_pl)  # noqa: E731
    nan = {s for s in range(len(lens)) if not ok(s)}
    for it in items:
        mem = [int(x) for x in it if x >= 0]
        ref = mem[0]
        ref_lim = pl[ref] if ok(ref) else -1
        for s in mem:
            if not ok(s) or pl[s] == 0:
                continue
            n = pl[s] // bs
            if pl[s] > ref_lim or not np.array_equal(tables[s, :n], tables[ref, :n]):
                nan.add(s)
    return sorted(nan)


def test_wrong_plans_give_nan_for_their_sequences_only():
    """Prefix lengths the tables do not back: the affected sequences' heads are
    NaN (by the rules of _expected_nan), every other sequence still matches the
    oracle."""
    bs, pb = 16, 6
    lens = np.array([200, 150, 120, 97, 300, 180, 96 + 1, 250] * 2)
    wl = _shared(32, 8, 64, bs, lens, 2, pb, "bf16", seed=7)
    plan = _plan(wl)
    kc, vc = oracle_caches(wl, 0)
    ref = oracle_decode(wl, 0, kc, vc)
    B, Hq, D = len(lens), wl.cfg.num_q_heads, wl.cfg.head_dim
    members = [int(x) for x in plan.items[0] if x >= 0]
    rs, other = members[0], members[1]
    cases = {
        "a member one block past the shared ones": (other, plan.prefix_len[other] + bs),
        "a member not a multiple of 16": (other, plan.prefix_len[other] - 8),
        "a member up to its last position": (other, int(lens[other])),
        "the reference one block further (its own blocks)": (rs, plan.prefix_len[rs] + bs),
        "the reference past its last position": (rs, int(lens[rs]) + bs),
    }
    saw_nan = False
    for what, (seq, bad_len) in cases.items():
        pl = plan.prefix_len.copy()
        pl[seq] = bad_len
        # the bound admits the larger length, so only the kernel's own checks can catch it
        mpl = max(plan.max_prefix_len, int(pl.max()))
        mpl = min(mpl, int(lens.max()))
        p2 = pkv.PrefixPlan(pl, plan.items, mpl)
        expect = _expected_nan(pl, lens, plan.items, wl.block_tables, bs, mpl)
        out = _run(wl, 0, p2, True)[0].reshape(B, Hq, D)
        got = bits_to_f64(out, "bf16")
        nan_seqs = sorted(set(np.argwhere(~np.isfinite(got))[:, 0].tolist()))
        assert nan_seqs == expect, f"{what}: NaN for {nan_seqs}, expected {expect}"
        for s_ in expect:
            assert np.all(np.isnan(got[s_])), f"{what}: sequence {s_} only partly NaN"
        keep = [i for i in range(B) if i not in expect]
        r, e = assert_parity(out[keep], ref[keep], "bf16", what)
        saw_nan |= bool(expect)
        print(f"{what}: NaN sequences {nan_seqs}; the others max|err| {e:.2e}", flush=True)
    assert saw_nan


def _agree_ratio(a_bits, b_bits, dtype):
    """|a - b| against the bound for two work splits of the same inputs: each
    probability is rounded to the 16-bit type against a running maximum that
    depends on the split (the decode tests' plan-agreement bound, 8u absolute)."""
    a, b = bits_to_f64(a_bits, dtype), bits_to_f64(b_bits, dtype)
    ulp = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -10
    u = 2.0 ** -9 if dtype == "bf16" else 2.0 ** -12
    return float((np.abs(a - b) / (8 * u + ulp * np.abs(b))).max())


@pytest.mark.parametrize("cid,pt", [(5, 0), (5, 256), (3, 0), (3, 512), (2, 128), (1, 16), (4, 256)])
def test_work_list(cid, pt):
    """Launching only the live partitions (the host's work list, short ones one
    wave per kv head): against the oracle, the pools bit-identical to the
    oracle's append, and the outputs within the plan-agreement bound of the
    full grid's, with and without shared prefixes."""
    wl = _wl5() if cid == 5 else workloads.build(cid)
    c = wl.cfg
    mcl = int(wl.context_lens.max())
    plans = [_plan(wl)]
    if plans[0].num_items:
        plans.append(pkv.PrefixPlan(np.zeros_like(plans[0].prefix_len), plans[0].items[:0], 0))
    kc, vc = oracle_caches(wl, 0)
    ref = oracle_decode(wl, 0, kc, vc)
    for plan in plans:
        pl = plan.prefix_len if plan.num_items else None
        work = pkv.decode_work_list(wl.context_lens, c.num_kv_heads, mcl, pt, pl)
        full = _run(wl, 0, plan, True, pt)
        listed = _run(wl, 0, plan, True, pt, work=work)
        assert np.array_equal(listed[1], kc) and np.array_equal(listed[2], vc), "pools"
        r, e = assert_parity(listed[0], ref, c.dtype, f"config {cid} partition {pt} items {plan.num_items}")
        agree = _agree_ratio(listed[0], full[0], c.dtype)
        waves = int(((work[:, 1].astype(np.int64) & 0xffffffff) >> 31).sum())
        print(f"config {cid} partition {pt} items {plan.num_items}: {len(work)} workgroups ({waves} in wave mode), "
              f"max|err| {e:.2e}, agreement with the full grid {agree:.3f}", flush=True)
        assert agree <= 1.0


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}q{s[1]}kv-d{s[2]}-bs{s[3]}-{s[4]}")
def test_work_list_shapes(shape):
    """Wave mode and the work list on every GQA size, both head dims, block
    sizes to 1024, forced partitions, with shared prefixes, fused and not."""
    Hq, Hkv, D, bs, dt, groups, pb = shape
    edges = [0, 1, 2, 17, bs, bs + 1, 2 * bs, 2 * bs + 1, 3 * bs + 1, pb * bs, pb * bs + 1, pb * bs + 2,
             (pb + 1) * bs + 1, (pb + 3) * bs + 5]
    lens = np.array([e for _ in range(groups) for e in edges])
    wl = _shared(Hq, Hkv, D, bs, lens, groups, pb, dt, seed=3)
    plan = _plan(wl)
    mcl = int(wl.context_lens.max())
    kc, vc = oracle_caches(wl, 0)
    ref = oracle_decode(wl, 0, kc, vc)
    for pt in (0, 16, 48, 512):
        work = pkv.decode_work_list(wl.context_lens, Hkv, mcl, pt, plan.prefix_len if plan.num_items else None)
        for fused in (False, True):
            out, kg, vg = _run(wl, 0, plan, fused, pt, work=work)
            if fused:
                assert np.array_equal(kg, kc) and np.array_equal(vg, vc)
            r, e = assert_parity(out, ref, dt, f"{shape} partition {pt} fused {fused} work list")
        print(f"{shape} partition {pt}: {len(work)} workgroups, max|err| {e:.2e}", flush=True)


def test_work_list_degenerate_sequences():
    """Empty sequences and lengths past the bound: partition 0 alone answers
    them (zeros, NaN), as in the full grid; the others agree with it."""
    wl = workloads.custom(16, 4, 64, 16, [0, 300, 1, 0, 2000, 17], "bf16", seed=2)
    lens = wl.context_lens.copy()
    lens[4] = 3000  # past max_context_len (the tables' 2000 tokens): NaN
    plan = _plan(wl)
    work = pkv.decode_work_list(lens, 4, 2000, 256)
    dw = upload(wl, layers=[0])
    d = dw.layers[0]
    poison_tails_gpu(wl, d)
    pkv.kv_append(d.k_new, d.v_new, dw.slots, d.k_cache, d.v_cache)
    lens_d = torch.from_numpy(lens).cuda()
    pl, items = _dev_plan(plan)
    outs = []
    for w in (None, torch.from_numpy(work).cuda()):
        outs.append(to_bits(pkv.paged_attn_decode_prefix(d.q, d.k_cache, d.v_cache, dw.tables, lens_d, wl.cfg.scale,
                                                         pl, items, 0, max_context_len=2000, partition_tokens=256,
                                                         work=w)))
    got = bits_to_f64(outs[1], "bf16")
    assert np.all(got[0] == 0) and np.all(got[3] == 0) and np.all(np.isnan(got[4]))
    assert np.array_equal(outs[0][[0, 3, 4]], outs[1][[0, 3, 4]])
    live = [1, 2, 5]
    assert _agree_ratio(outs[1][live], outs[0][live], "bf16") <= 1.0

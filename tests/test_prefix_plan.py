"""pkv_decode_prefix_plan (host): grouping sequences that share leading blocks
into prefix items, checked against the tables themselves, plus the prefix
decode entry point's argument checks (no GPU needed)."""
import ctypes

import numpy as np
import pytest

import paged_kv_cache_448_amd as pkv
import workloads

OK, E_NULL, E_SHAPE, E_UNSUPPORTED = 0, -1, -2, -3


def members_per_item(head_dim, group):
    cg = min(2 if head_dim == 64 else 1, group)
    return cg * 16 // group


def check_plan(plan, tables, lens, bs, per_item):
    """Every property the decode kernel relies on, by brute force over the rows."""
    B = len(lens)
    pl = plan.prefix_len
    assert pl.shape == (B,) and plan.items.ndim == 2 and plan.items.shape[1] == 16
    seen = np.zeros(B, dtype=np.int64)
    for it in plan.items:
        mem = [int(x) for x in it if x >= 0]
        assert list(it[:len(mem)]) == mem and all(x == -1 for x in it[len(mem):]), "members first, -1 pads"
        assert 2 <= len(mem) <= per_item
        assert len(set(mem)) == len(mem)
        ref = mem[0]
        for s in mem:
            seen[s] += 1
            n = pl[s] // bs
            assert pl[s] > 0 and pl[s] % bs == 0
            assert pl[s] <= lens[s] - 1, "the token of this step is never in the prefix"
            assert np.array_equal(tables[s, :n], tables[ref, :n]), f"seq {s} does not share {n} blocks with {ref}"
        assert pl[ref] == max(pl[s] for s in mem[1:]), "the reference covers exactly the longest member"
    assert np.all(seen[pl > 0] == 1), "every sequence with a prefix is in exactly one item"
    assert np.all(pl[seen == 0] == 0)
    assert plan.max_prefix_len == (int(pl.max()) if B else 0)


def expected_shared(wl):
    """Shared tokens per sequence by the workload's own rule (its shared blocks)."""
    c = wl.cfg
    out = np.zeros(len(wl.context_lens), dtype=np.int64)
    for i, L in enumerate(wl.context_lens.astype(np.int64)):
        out[i] = c.block_size * sum(1 for j in range(min(c.prefix_blocks, -(-int(L) // c.block_size)))
                                    if c.block_size * (j + 1) <= L - 1)
    return out


def shared_workload(Hq, Hkv, D, bs, lens, groups, prefix_blocks, dtype="bf16", seed=0):
    cfg = workloads.Config(0, "custom-shared", 1, len(lens), Hq, Hkv, D, bs, dtype, "fixed",
                           fixed_lens=tuple(int(x) for x in lens), prefix_groups=groups, prefix_blocks=prefix_blocks)
    return workloads.build_config(cfg, seed=seed, poison=False)


def test_cb_step_workload():
    wl = workloads.build(5, num_layers=1)
    c = wl.cfg
    plan = pkv.decode_prefix_plan(wl.block_tables, wl.context_lens, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                  c.block_size)
    per = members_per_item(c.head_dim, c.group)
    check_plan(plan, wl.block_tables, wl.context_lens, c.block_size, per)
    exp = expected_shared(wl)
    assert np.all(plan.prefix_len <= exp), "never more than the workload shares"
    # the private blocks are distinct, so only a reference whose item shares
    # less than it could is cut short
    short = plan.prefix_len < exp
    refs = set(int(it[0]) for it in plan.items)
    assert all(i in refs or exp[i] == 0 for i in np.flatnonzero(short))
    assert plan.prefix_len.sum() >= 0.98 * exp.sum()
    # items fill up to the member limit within each group of sharers
    assert plan.num_items <= -(-int((exp > 0).sum()) // per) + c.prefix_groups


@pytest.mark.parametrize("shape", [(32, 8, 64, 16), (16, 16, 128, 16), (64, 4, 64, 32), (8, 4, 128, 64),
                                   (16, 2, 64, 256), (16, 1, 128, 16)])
def test_shapes_and_block_edges(shape):
    Hq, Hkv, D, bs = shape
    edges = [0, 1, 2, bs, bs + 1, bs + 2, 2 * bs, 2 * bs + 1, 3 * bs + 1, 5 * bs, 5 * bs + 1, 9 * bs + 7, 40 * bs]
    lens = np.array(edges * 4)
    wl = shared_workload(Hq, Hkv, D, bs, lens, 4, 6)
    plan = pkv.decode_prefix_plan(wl.block_tables, wl.context_lens, Hq, Hkv, D, bs)
    per = members_per_item(D, Hq // Hkv)
    check_plan(plan, wl.block_tables, wl.context_lens, bs, per)
    assert np.all(plan.prefix_len <= expected_shared(wl))
    if per >= 2:
        assert plan.num_items > 0
    else:
        assert plan.num_items == 0, "one member per item: nothing to share"


def test_random_prefix_trees():
    """Tables built as a tree of shared prefixes (each sequence copies a random
    number of leading blocks from a random earlier one), many seeds."""
    for seed in range(40):
        rng = np.random.default_rng(seed)
        B, M, bs = int(rng.integers(1, 60)), 24, 16
        lens = rng.integers(0, M * bs + 1, size=B).astype(np.int32)
        tables = np.zeros((B, M), dtype=np.int32)
        nxt = 0
        for i in range(B):
            k = 0
            if i and rng.random() < 0.8:
                j = int(rng.integers(0, i))
                k = int(rng.integers(0, M + 1))
                tables[i, :k] = tables[j, :k]
            tables[i, k:] = np.arange(nxt, nxt + M - k)
            nxt += M - k
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = 2
        D = int(rng.choice([64, 128]))
        plan = pkv.decode_prefix_plan(tables, lens, G * Hkv, Hkv, D, bs)
        check_plan(plan, tables, lens, bs, members_per_item(D, G))


def test_no_sharing_and_degenerate():
    tables = np.arange(40, dtype=np.int32).reshape(8, 5)
    lens = np.array([0, 1, 17, 80, 33, 2, 16, 79], dtype=np.int32)
    plan = pkv.decode_prefix_plan(tables, lens, 8, 2, 64, 16)
    assert plan.num_items == 0 and plan.max_prefix_len == 0 and not plan.prefix_len.any()
    # identical rows but every length at most one block plus the last token's position
    same = np.zeros((4, 5), dtype=np.int32)
    plan = pkv.decode_prefix_plan(same, np.array([0, 1, 16, 16], dtype=np.int32), 8, 2, 64, 16)
    assert plan.num_items == 0
    plan = pkv.decode_prefix_plan(same, np.array([17, 17, 0, 1], dtype=np.int32), 8, 2, 64, 16)
    assert plan.num_items == 1 and list(plan.prefix_len) == [16, 16, 0, 0]
    plan = pkv.decode_prefix_plan(np.zeros((0, 5), np.int32), np.zeros(0, np.int32), 8, 2, 64, 16)
    assert plan.num_items == 0


def _plan_raw(tables, lens, Hq=8, Hkv=2, D=64, bs=16, cap=None, null_items=False):
    B, M = tables.shape
    pl = np.zeros(B, dtype=np.int32)
    items = np.zeros((max(B // 2 + 1, 1), 16), dtype=np.int32)
    n, lg = ctypes.c_int32(), ctypes.c_int32()
    return pkv.lib().pkv_decode_prefix_plan(tables.ctypes.data, M, lens.ctypes.data, B, Hq, Hkv, D, bs,
                                            pl.ctypes.data, None if null_items else items.ctypes.data,
                                            items.shape[0] if cap is None else cap, ctypes.byref(n),
                                            ctypes.byref(lg))


def test_plan_errors():
    tables = np.zeros((6, 4), dtype=np.int32)
    lens = np.full(6, 40, dtype=np.int32)
    assert _plan_raw(tables, lens) == OK
    assert _plan_raw(tables, lens, cap=0) == E_SHAPE, "items need room"
    assert _plan_raw(tables, lens, null_items=True) == E_NULL
    assert _plan_raw(tables, lens, Hq=6, Hkv=4) == E_SHAPE
    assert _plan_raw(tables, lens, bs=24) == E_UNSUPPORTED
    assert _plan_raw(tables, lens, D=96) == E_UNSUPPORTED
    # 16 members at G = 1, head_dim 128: six identical rows make one item
    B = 6
    pl = np.zeros(B, dtype=np.int32)
    items = np.zeros((4, 16), dtype=np.int32)
    n, lg = ctypes.c_int32(), ctypes.c_int32()
    assert pkv.lib().pkv_decode_prefix_plan(tables.ctypes.data, 4, lens.ctypes.data, B, 2, 2, 128, 16,
                                            pl.ctypes.data, items.ctypes.data, 4, ctypes.byref(n),
                                            ctypes.byref(lg)) == OK
    assert n.value == 1 and lg.value == 32 and sorted(items[0, :6]) == list(range(6))


def _decode_prefix(**kw):
    a = dict(q=16, kn=None, vn=None, sm=None, kc=16, vc=16, bt=16, mb=4, cl=16, mcl=64, scale=0.125, out=16, B=2,
             Hq=4, Hkv=2, D=64, bs=16, N=8, dt=0, pl=16, items=16, ni=1, mpl=32, ws=None, wsb=0, pt=0, work=None, nw=0)
    a.update(kw)
    p = lambda x: ctypes.c_void_p(x) if x is not None else None  # noqa: E731
    return pkv.lib().pkv_paged_attn_decode_prefix(
        p(a["q"]), p(a["kn"]), p(a["vn"]), p(a["sm"]), p(a["kc"]), p(a["vc"]), p(a["bt"]), a["mb"], p(a["cl"]),
        a["mcl"], ctypes.c_float(a["scale"]), p(a["out"]), a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["N"],
        a["dt"], p(a["pl"]), p(a["items"]), a["ni"], a["mpl"], p(a["ws"]), ctypes.c_size_t(a["wsb"]), a["pt"],
        None, p(a["work"]), a["nw"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(pl=None), E_NULL), (dict(items=None), E_NULL), (dict(ni=-1), E_SHAPE), (dict(mpl=-16), E_SHAPE),
    (dict(mpl=65), E_SHAPE), (dict(D=96), E_UNSUPPORTED), (dict(Hq=6, Hkv=4), E_SHAPE),
    (dict(ws=None, wsb=0), -4), (dict(nw=-1), E_SHAPE), (dict(nw=3, work=None), E_NULL),
])
def test_decode_prefix_rejects_before_launch(kw, status):
    assert _decode_prefix(**kw) == status


def test_decode_prefix_workspace():
    # prefix chunks add slots: the plain plan needs none here, the prefix one does
    plain = pkv.decode_workspace_bytes(64, 32, 8, 64, 16, 2048)
    assert plain == 0
    w = pkv.decode_prefix_workspace_bytes(64, 32, 8, 64, 16, 2048, 512)
    rows = 64 * 32 * (1 + 2)  # one pass + two prefix chunks of 256 tokens
    align = lambda n: (n + 255) // 256 * 256  # noqa: E731
    assert w == align(rows * 64 * 4) + 2 * align(rows * 4)
    assert pkv.decode_prefix_workspace_bytes(64, 32, 8, 64, 16, 2048, 0) == plain
    # chunk = half the longest prefix in multiples of 16, clamped to [64, 1024]
    for mpl, chunks in ((16, 1), (64, 1), (100, 2), (256, 2), (257, 2), (2400, 3), (4096, 4), (8000, 8)):
        w = pkv.decode_prefix_workspace_bytes(2, 4, 2, 64, 16, 8192, mpl, 8192)
        rows = 2 * 4 * (1 + chunks)
        assert w == align(rows * 64 * 4) + 2 * align(rows * 4), (mpl, chunks)


def _decode_entries(work, Hkv, nw):
    """(seq, part, kv head, wave mode) per workgroup, wave-mode entries expanded to their heads."""
    out = []
    for s_, y in np.asarray(work, dtype=np.int64):
        y &= 0xffffffff
        part, h, mode = int(y & 0xffff), int((y >> 16) & 0x7fff), int(y >> 31)
        if s_ < 0:
            assert y == 0, "padding entries are (-1, 0)"
            continue
        heads = range(h, min(h + nw, Hkv)) if mode else [h]
        out += [(int(s_), part, hh, mode) for hh in heads]
    return out


def test_work_list_covers_live_partitions_once():
    """Every sequence's partition 0 and each partition that holds tokens, for
    every kv head, once; nothing past a context's end; partitions of at most
    256 tokens in wave mode (one wave per head), longer ones a workgroup per head."""
    for seed in range(20):
        rng = np.random.default_rng(seed)
        B = int(rng.integers(1, 300))
        lens = rng.integers(0, 6000, size=B).astype(np.int32)
        lens[rng.random(B) < 0.05] = 0
        Hkv = int(rng.choice([1, 2, 8, 12]))
        mcl = int(lens.max()) if B else 0
        pt_req = int(rng.choice([0, 256, 1536]))
        pt = pkv.plan_partition(B, Hkv, 16, mcl) if pt_req == 0 else pt_req
        part_tokens = pt if pt and pt < mcl else max(16, (mcl + 15) // 16 * 16)
        nparts = max(1, -(-mcl // part_tokens))
        nw = 8 if nparts == 1 or part_tokens > 4096 else 4
        pl = None
        if seed % 2:
            pl = (rng.integers(0, 40, size=B) * 16).astype(np.int32)
            pl = np.where(pl <= lens - 1, pl, 0).astype(np.int32)
        work = pkv.decode_work_list(lens, Hkv, mcl, pt_req, pl)
        assert len(work) % 8 == 0, "eight equal ranges"
        ent = _decode_entries(work, Hkv, nw)
        got = [(s_, part, h) for s_, part, h, _ in ent]
        assert len(set(got)) == len(got), seed
        expect = set()
        for i, L in enumerate(lens):
            p0 = 0 if pl is None else int(pl[i])
            n = max(1, -(-(int(L) - p0) // part_tokens)) if L > 0 else 1
            expect |= {(i, k, h) for k in range(n) for h in range(Hkv)}
        assert set(got) == expect, seed
        for s_, part, h, mode in ent:
            L = int(lens[s_])
            p0 = 0 if pl is None else int(pl[s_])
            toks = max(0, min(part_tokens, L - p0 - part * part_tokens)) if L > 0 else 0
            assert mode == (toks <= 256), (seed, s_, part, toks, mode)


def test_work_list_balances_xcds():
    lens = np.array([5000, 100, 3000, 3000, 20, 1536, 1537, 4000] * 8, dtype=np.int32)
    work = pkv.decode_work_list(lens, 8, 5000, 1536)
    n = len(work) // 8
    loads, seqs = [], []
    for g in range(8):
        ent = _decode_entries(work[g * n:(g + 1) * n], 8, 4)
        seqs.append({s_ for s_, _, _, _ in ent})
        loads.append(sum(min(1536, int(lens[s_]) - part * 1536) for s_, part, _, _ in ent) // 8)
    for g in range(8):
        for o in range(g + 1, 8):
            assert not seqs[g] & seqs[o], "a sequence on one XCD"
    assert max(loads) - min(loads) <= int(lens.max()), loads


def test_work_list_small():
    w = pkv.decode_work_list(np.array([5], np.int32), 1, 16, 0)
    # one 5-token partition: wave mode (bit 31), kv head 0
    assert [tuple(int(v) for v in x) for x in w] == [(0, -(1 << 31))] + [(-1, 0)] * 7
    # equal loads: the group with fewer entries, so the two land on two XCDs
    w = pkv.decode_work_list(np.array([0, 0], np.int32), 2, 0, 0)
    assert [int(x[0]) for x in w] == [0, 1] + [-1] * 6


def test_work_list_errors():
    lens = np.array([100, 2000], dtype=np.int32)
    w = np.zeros((1, 2), dtype=np.int32)
    n = ctypes.c_int32()
    assert pkv.lib().pkv_decode_work_list(lens.ctypes.data, None, 2, 2, 2000, 256, w.ctypes.data, 1,
                                          ctypes.byref(n)) == E_SHAPE
    assert pkv.lib().pkv_decode_work_list(lens.ctypes.data, None, 2, 2, 2000, 24, w.ctypes.data, 1,
                                          ctypes.byref(n)) == E_SHAPE
    assert pkv.lib().pkv_decode_work_list(None, None, 2, 2, 2000, 256, w.ctypes.data, 1, ctypes.byref(n)) == E_NULL

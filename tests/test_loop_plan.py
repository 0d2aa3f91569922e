"""Continuous-batching loop, host side (no GPU): the step plans, the host
allocator driven through a whole plan, and the oracle replay pinned against the
paged-decode oracle.
"""
import numpy as np
import pytest

import paged_kv_cache_448_amd as pkv
from oracle import alloc_check
from oracle import attention as oracle_attn
from oracle.loop import LoopReplay
from oracle.numerics import bits_to_f64
from workloads import loop as wl_loop

CFG = wl_loop.LOOP_CONFIGS["tiny-loop"]


def _plan(steps=80, seed=7):
    return wl_loop.plan(CFG, seed, steps)


def test_plan_invariants():
    reqs, steps = _plan()
    admitted_at, first_run, last_run, runs = {}, {}, {}, {}
    reserved = 0
    for st in steps:
        for rid in st.admit:
            admitted_at[rid] = st.index
            assert reqs[rid].arrival <= st.index
        assert len(st.run) <= CFG.max_batch
        assert st.run == sorted(st.run)
        for rid in st.run:
            first_run.setdefault(rid, st.index)
            last_run[rid] = st.index
            runs[rid] = runs.get(rid, 0) + 1
        live = set(st.run)
        reserved = sum(wl_loop.blocks_for(reqs[r].prompt_len + reqs[r].gen_len, CFG.block_size) for r in live)
        assert reserved <= CFG.num_blocks
        for rid in st.finish:
            assert rid in live and runs[rid] == reqs[rid].gen_len
    # first come, first served; every admitted request runs gen_len consecutive steps from its admission
    order = sorted(admitted_at, key=lambda r: (admitted_at[r], r))
    assert order == sorted(admitted_at)
    for rid, s0 in admitted_at.items():
        assert first_run[rid] == s0
        if rid in set().union(*[set(s.finish) for s in steps]):
            assert last_run[rid] - s0 + 1 == reqs[rid].gen_len
    assert len(admitted_at) == CFG.num_requests  # the tiny plan drains the whole stream


def test_plan_is_deterministic_and_seeded():
    a = _plan(seed=7)[1]
    b = _plan(seed=7)[1]
    c = _plan(seed=8)[1]
    assert [(s.admit, s.run, s.finish) for s in a] == [(s.admit, s.run, s.finish) for s in b]
    assert [(s.admit, s.run, s.finish) for s in a] != [(s.admit, s.run, s.finish) for s in c]


def test_host_allocator_runs_the_plan():
    """The library's host allocator through every step: no NOMEM, valid tables and slots,
    and every block back in the pool at the end."""
    reqs, steps = _plan()
    alloc = pkv.BlockAllocator(CFG.num_blocks, CFG.block_size, shuffle_seed=3)
    bs = CFG.block_size
    live = set()
    for st in steps:
        for rid in st.admit:
            alloc.add_seq(rid, reqs[rid].prompt_len)
            live.add(rid)
        if st.run:
            before = {rid: alloc.context_len(rid) for rid in st.run}
            slots = alloc.append_slots(st.run)
            M = max(1, -(-max(alloc.context_len(r) for r in st.run) // bs))
            tables, lens = alloc.block_tables(st.run, M, pad_value=-1)
            alloc_check.check_tables(tables, lens, num_blocks=CFG.num_blocks, block_size=bs, pad_value=-1)
            for i, rid in enumerate(st.run):
                assert lens[i] == before[rid] + 1
                assert slots[i] == alloc_check.slot_of(tables, i, int(lens[i]) - 1, bs)
            assert len(set(slots.tolist())) == len(slots)
        for rid in st.finish:
            alloc.free_seq(rid)
            live.discard(rid)
        in_use = sum(alloc_check.blocks_needed(alloc.context_len(r), bs) for r in live)
        assert alloc.num_free == CFG.num_blocks - in_use
    assert not live and alloc.num_free == CFG.num_blocks


def test_replay_matches_paged_oracle():
    """One sequence's replayed step equals the paged-decode oracle on the same context laid
    out in a shuffled pool: the replay drops the pool, not the arithmetic."""
    rng = np.random.default_rng(5)
    Hq, Hkv, D, bs = CFG.num_q_heads, CFG.num_kv_heads, CFG.head_dim, CFG.block_size
    P = 37
    k_p, v_p = wl_loop.prompt_values(CFG, 5, 0, 0, P)
    q, k_n, v_n = wl_loop.step_values(CFG, 5, 0, 0, 1)
    rep = LoopReplay(Hq, Hkv, D, CFG.dtype, CFG.scale)
    rep.admit(0, 0, k_p, v_p)
    got = rep.step(0, [0], q, k_n, v_n)
    L = P + 1
    nblk = -(-L // bs)
    N = nblk + 3
    table = rng.permutation(N)[:nblk]
    kc = np.zeros((N, Hkv, bs, D), dtype=np.uint16)
    vc = np.zeros_like(kc)
    ks = np.concatenate([k_p, k_n], axis=0)
    vs = np.concatenate([v_p, v_n], axis=0)
    for t in range(L):
        kc[table[t // bs], :, t % bs] = ks[t]
        vc[table[t // bs], :, t % bs] = vs[t]
    ref = oracle_attn.decode(q, kc.ravel(), vc.ravel(), table[None], np.array([L]), CFG.scale, dtype=CFG.dtype,
                             num_blocks=N, num_kv_heads=Hkv, block_size=bs)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_replay_first_token_of_empty_prompt_is_its_v():
    """A request with no prompt: its first step attends over the appended token alone, so each
    q head outputs that token's V for its kv head, exactly."""
    Hq, Hkv, D = CFG.num_q_heads, CFG.num_kv_heads, CFG.head_dim
    rep = LoopReplay(Hq, Hkv, D, CFG.dtype, CFG.scale)
    rep.admit(3, 1, np.zeros((0, Hkv, D), np.uint16), np.zeros((0, Hkv, D), np.uint16))
    q, k, v = wl_loop.step_values(CFG, 9, 4, 1, 1)
    out = rep.step(1, [3], q, k, v)
    vv = bits_to_f64(v[0], CFG.dtype)
    for h in range(Hq):
        assert np.array_equal(out[0, h], vv[h // (Hq // Hkv)])


@pytest.mark.parametrize("bad", ["drop-prompt", "skip-append"])
def test_replay_pins_catch_planted_mistakes(bad):
    """A replay that forgets the prompt or the appended token disagrees with the paged oracle."""
    Hq, Hkv, D, bs = CFG.num_q_heads, CFG.num_kv_heads, CFG.head_dim, CFG.block_size
    P = 20
    k_p, v_p = wl_loop.prompt_values(CFG, 5, 1, 0, P)
    q, k_n, v_n = wl_loop.step_values(CFG, 5, 1, 0, 1)
    rep = LoopReplay(Hq, Hkv, D, CFG.dtype, CFG.scale)
    if bad == "drop-prompt":
        rep.admit(0, 0, k_p[:0], v_p[:0])
        got = rep.step(0, [0], q, k_n, v_n)
    else:
        rep.admit(0, 0, k_p, v_p)
        kc, vc = rep.context(0, 0)
        got = np.stack([oracle_attn.attend(bits_to_f64(q[0, h:h + 1], CFG.dtype),
                                           bits_to_f64(kc[:, h // (Hq // Hkv)], CFG.dtype),
                                           bits_to_f64(vc[:, h // (Hq // Hkv)], CFG.dtype),
                                           float(np.float32(CFG.scale)))[0] for h in range(Hq)])[None]
    L = P + 1
    table = np.arange(-(-L // bs))
    kc = np.zeros((len(table), Hkv, bs, D), dtype=np.uint16)
    vc = np.zeros_like(kc)
    ks = np.concatenate([k_p, k_n], axis=0)
    vs = np.concatenate([v_p, v_n], axis=0)
    for t in range(L):
        kc[t // bs, :, t % bs] = ks[t]
        vc[t // bs, :, t % bs] = vs[t]
    ref = oracle_attn.decode(q, kc.ravel(), vc.ravel(), table[None], np.array([L]), CFG.scale, dtype=CFG.dtype,
                             num_blocks=len(table), num_kv_heads=Hkv, block_size=bs)
    assert not np.allclose(got, ref, rtol=0, atol=1e-6)


def test_token_values_depend_only_on_the_prefix():
    lc = wl_loop.LOOP_CONFIGS["tiny-prefix-loop"]
    a = wl_loop.prompt_tokens(lc, 3, 0, 60)
    b = wl_loop.prompt_tokens(lc, 3, 3, 60)       # same group (3 groups): same 40-token prefix
    c = wl_loop.prompt_tokens(lc, 3, 1, 60)       # another group
    assert np.array_equal(a[:40], b[:40]) and not np.array_equal(a[:40], c[:40])
    ka, va = wl_loop.token_values(lc, 3, a, 1)
    kb, vb = wl_loop.token_values(lc, 3, b, 1)
    first = int(np.argmax(a != b))
    assert first >= 40
    assert np.array_equal(ka[:first], kb[:first]) and np.array_equal(va[:first], vb[:first])
    assert not np.array_equal(ka[first], kb[first])

"""Continuous-batching decode loop on the GPU against the oracle replay.

The GPU side is DecodeLoop: the library's host allocator (admissions, one slot
per running sequence per step, frees, block reuse across steps) and its kernels
(kv_append of each prompt, one fused append + decode launch per layer and
step).  The oracle side keeps each sequence's context as a plain array.  Every
step's outputs must agree within |err| <= 1e-2 + 1e-2 |ref|, and the K/V a live
sequence holds in the pools must equal its replayed context bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_harness import assert_parity, to_bits, to_dev
from oracle.loop import LoopReplay
from paged_kv_cache_448_amd.loop import DecodeLoop
from workloads import loop as wl_loop

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", [7, 21])
def test_loop_matches_replay(seed):
    lc = wl_loop.LOOP_CONFIGS["tiny-loop"]
    reqs, steps = wl_loop.plan(lc, seed, 120)
    gpu = DecodeLoop(lc, shuffle_seed=seed)
    rep = LoopReplay(lc.num_q_heads, lc.num_kv_heads, lc.head_dim, lc.dtype, lc.scale)
    reused = set()
    ever_held = set()
    worst = 0.0
    for st in steps:
        if st.admit:
            lens_p = [reqs[rid].prompt_len for rid in st.admit]
            per_layer = []
            for layer in range(lc.num_layers):
                ks, vs = [], []
                for rid, P in zip(st.admit, lens_p):
                    k, v = wl_loop.prompt_values(lc, seed, rid, layer, P)
                    rep.admit(rid, layer, k, v)
                    ks.append(k)
                    vs.append(v)
                T = sum(lens_p)
                shape = (T, lc.num_kv_heads, lc.head_dim)
                per_layer.append((to_dev(np.concatenate(ks), lc.dtype, shape), to_dev(np.concatenate(vs), lc.dtype, shape)))
            gpu.admit(st.admit, lens_p, lambda layer, cached: per_layer[layer])
        if not st.run:
            continue
        B = len(st.run)
        vals = [wl_loop.step_values(lc, seed, st.index, layer, B) for layer in range(lc.num_layers)]
        dev = [tuple(to_dev(a, lc.dtype) for a in v) for v in vals]
        outs = [torch.empty((B, lc.num_q_heads, lc.head_dim), dtype=gpu.dtype, device="cuda")
                for _ in range(lc.num_layers)]
        gpu.decode_step(st.run, lambda layer: dev[layer], outs)
        torch.cuda.synchronize()
        for layer in range(lc.num_layers):
            q, k, v = vals[layer]
            ref = rep.step(layer, st.run, q, k, v)
            r, _ = assert_parity(to_bits(outs[layer]), ref, lc.dtype, f"seed {seed} step {st.index} layer {layer}")
            worst = max(worst, r)
        # block reuse: note blocks that held an earlier (finished) sequence's tokens
        tables, lens = gpu.alloc.block_tables(st.run, gpu.max_blocks, pad_value=-1)
        for i in range(B):
            blocks = set(tables[i, :-(-int(lens[i]) // lc.block_size)].tolist())
            reused |= blocks & ever_held
        if st.index % 7 == 0:
            for rid in st.run[:2]:
                for layer in range(lc.num_layers):
                    kd, vd = gpu.gather(rid, layer)
                    kr, vr = rep.context(rid, layer)
                    assert np.array_equal(to_bits(kd), kr) and np.array_equal(to_bits(vd), vr), (rid, layer)
        for rid in st.finish:
            t, ln = gpu.alloc.block_tables([rid], gpu.max_blocks, pad_value=-1)
            ever_held |= set(t[0, :-(-int(ln[0]) // lc.block_size)].tolist())
            gpu.finish(rid)
            rep.finish(rid, lc.num_layers)
    assert gpu.alloc.num_free == lc.num_blocks and gpu.alloc.num_seqs == 0
    assert reused, "the plan should hand freed blocks to later sequences"
    print(f"seed {seed}: {sum(len(s.run) for s in steps)} decode tokens over {len(steps)} steps, "
          f"{len(reused)} blocks reused, worst ratio to tolerance {worst:.3f}", flush=True)


@pytest.mark.parametrize("seed", [3])
def test_prefix_cached_loop_matches_replay(seed):
    """Prompts given as token ids in groups with a common prefix: the allocator shares the
    prefix's full blocks and only the other positions are written, yet every output and every
    live sequence's pooled K/V equal the replay of the sequence's own full context (whose K/V
    rows depend only on the token prefix, as a model's do)."""
    lc = wl_loop.LOOP_CONFIGS["tiny-prefix-loop"]
    reqs, steps = wl_loop.plan(lc, seed, 120)
    gpu = DecodeLoop(lc, shuffle_seed=seed)
    rep = LoopReplay(lc.num_q_heads, lc.num_kv_heads, lc.head_dim, lc.dtype, lc.scale)
    total_cached = 0
    for st in steps:
        if st.admit:
            lens_p = [reqs[rid].prompt_len for rid in st.admit]
            toks = [wl_loop.prompt_tokens(lc, seed, rid, P) for rid, P in zip(st.admit, lens_p)]
            full = [[wl_loop.token_values(lc, seed, t, layer) for layer in range(lc.num_layers)] for t in toks]
            for rid, kv in zip(st.admit, full):
                for layer in range(lc.num_layers):
                    rep.admit(rid, layer, *kv[layer])

            def prompt_kv(layer, cached):
                ks = np.concatenate([full[i][layer][0][c:] for i, c in enumerate(cached)])
                vs = np.concatenate([full[i][layer][1][c:] for i, c in enumerate(cached)])
                shape = (len(ks), lc.num_kv_heads, lc.head_dim)
                return to_dev(ks, lc.dtype, shape), to_dev(vs, lc.dtype, shape)

            cached = gpu.admit(st.admit, lens_p, prompt_kv, token_ids=toks)
            total_cached += sum(cached)
        if not st.run:
            continue
        B = len(st.run)
        vals = [wl_loop.step_values(lc, seed, st.index, layer, B) for layer in range(lc.num_layers)]
        dev = [tuple(to_dev(a, lc.dtype) for a in v) for v in vals]
        outs = [torch.empty((B, lc.num_q_heads, lc.head_dim), dtype=gpu.dtype, device="cuda")
                for _ in range(lc.num_layers)]
        gpu.decode_step(st.run, lambda layer: dev[layer], outs)
        torch.cuda.synchronize()
        for layer in range(lc.num_layers):
            q, k, v = vals[layer]
            ref = rep.step(layer, st.run, q, k, v)
            assert_parity(to_bits(outs[layer]), ref, lc.dtype, f"seed {seed} step {st.index} layer {layer}")
        for rid in st.run:
            for layer in range(lc.num_layers):
                kd, vd = gpu.gather(rid, layer)
                kr, vr = rep.context(rid, layer)
                assert np.array_equal(to_bits(kd), kr) and np.array_equal(to_bits(vd), vr), (st.index, rid, layer)
        for rid in st.finish:
            gpu.finish(rid)
            rep.finish(rid, lc.num_layers)
    assert total_cached > 0, "the groups' prefixes should have been shared"
    assert gpu.prefix_steps > 0, "some steps' decode should have read shared prefixes once per prefix item"
    assert gpu.alloc.num_free == lc.num_blocks
    print(f"seed {seed}: {total_cached} prompt tokens served from shared blocks; {gpu.prefix_steps} steps "
          f"decoded with prefix items", flush=True)

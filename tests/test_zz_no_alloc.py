"""The allocation-free decode entry point, pkv_paged_attn_decode_noalloc, against
pkv_paged_attn_decode with a caller-provided workspace.

Workload: the long-context batch (16 sequences of 4096-8192 tokens, block size
256), whose automatic plan splits every context, so the partial states go through
the library's per-GPU device scratch and the merge pass.  Two calls in a row, the
second on a smaller input (the first five sequences, a shorter bound): each is
bit-identical to the workspace call on the same input and within the decode
tolerance of the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_448_amd as pkv
import workloads
from gpu_harness import assert_parity, oracle_caches, oracle_decode, poison_tails_gpu, to_bits, upload

pytestmark = pytest.mark.gpu


def _setup():
    wl = workloads.build(3)
    dw = upload(wl, layers=[0])
    d = dw.layers[0]
    poison_tails_gpu(wl, d)
    pkv.kv_append(d.k_new, d.v_new, dw.slots, d.k_cache, d.v_cache)
    return wl, dw, d


def _pair(wl, d, q, tables, lens, mcl):
    c = wl.cfg
    ws = torch.empty(max(pkv.decode_workspace_bytes(q.shape[0], c.num_q_heads, c.num_kv_heads, c.head_dim,
                                                    c.block_size, mcl), 256), dtype=torch.uint8, device=q.device)
    ref = pkv.paged_attn_decode(q, d.k_cache, d.v_cache, tables, lens, c.scale, max_context_len=mcl, workspace=ws)
    out = torch.full_like(q, float("nan"))
    pkv.paged_attn_decode_noalloc(q, d.k_cache, d.v_cache, tables, lens, c.scale, out, max_context_len=mcl)
    torch.cuda.synchronize()
    return to_bits(ref), to_bits(out)


def test_noalloc_equals_workspace_call_twice_second_smaller():
    wl, dw, d = _setup()
    c = wl.cfg
    kc, vc = oracle_caches(wl, 0)
    lens = wl.context_lens
    B = len(lens)
    mcl = int(lens.max())
    assert pkv.plan_partition(B, c.num_kv_heads, c.block_size, mcl) > 0, "the workload must take the split path"
    ref, out = _pair(wl, d, d.q, dw.tables, dw.lens, mcl)
    assert np.array_equal(out, ref), "first call differs from the workspace call"
    assert_parity(out, oracle_decode(wl, 0, kc, vc), c.dtype, "first call vs oracle")
    print(f"call 1: {B} sequences, max_context_len {mcl}: bit-identical", flush=True)

    n = 5
    mcl2 = int(lens[:n].max())
    assert mcl2 < mcl and pkv.plan_partition(n, c.num_kv_heads, c.block_size, mcl2) > 0
    q2, t2, l2 = d.q[:n].contiguous(), dw.tables[:n].contiguous(), dw.lens[:n].contiguous()
    ref2, out2 = _pair(wl, d, q2, t2, l2, mcl2)
    assert np.array_equal(out2, ref2), "second (smaller) call differs from the workspace call"
    assert_parity(out2, oracle_decode(wl, 0, kc, vc, seqs=list(range(n))), c.dtype, "second call vs oracle")
    print(f"call 2: {n} sequences, max_context_len {mcl2}: bit-identical", flush=True)


def test_noalloc_refuses_plans_beyond_the_scratch():
    # 4096 sequences of up to 8192 tokens, 32 q heads of 128 dims: the split
    # plan's partial states need far more than 16 MiB; refused before any launch
    dummy = torch.empty(64, dtype=torch.bfloat16, device="cuda")
    p = dummy.data_ptr()
    st = pkv.lib().pkv_paged_attn_decode_noalloc(p, p, p, p, 32, p, 8192, 0.1, p, 4096, 32, 8, 128, 256, 1 << 16, 0,
                                                 None)
    assert st == -4  # PKV_E_WORKSPACE

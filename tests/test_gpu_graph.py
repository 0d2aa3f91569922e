"""The append + decode step captured in a HIP graph (through torch) and replayed:
every replay must equal the eager result bit for bit, with the program's own
eager work and synchronisations between replays."""
import numpy as np
import pytest
import torch

import paged_kv_cache_448_amd as pkv
import workloads
from gpu_harness import to_bits, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cid,impl", [(2, "mfma"), (2, "simt"), (3, "mfma")])
def test_graph_replays_match_eager(cid, impl):
    wl = workloads.build(cid, poison=False)
    c = wl.cfg
    dw = upload(wl)
    d = dw.layers[0]
    B = len(wl.context_lens)
    mcl = int(wl.context_lens.max())
    ws = torch.empty(max(pkv.decode_workspace_bytes(B, c.num_q_heads, c.num_kv_heads, c.head_dim, c.block_size,
                                                    mcl), 256), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d.q)

    def step():
        pkv.kv_append(d.k_new, d.v_new, dw.slots, d.k_cache, d.v_cache)
        pkv.paged_attn_decode(d.q, d.k_cache, d.v_cache, dw.tables, dw.lens, c.scale, out, max_context_len=mcl,
                              workspace=ws, impl=impl)

    step()
    torch.cuda.synchronize()
    eager = to_bits(out).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.fill_(0)                       # eager work between replays
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(out), eager), f"replay {rep} differs from eager"

"""KV byte accounting against the vLLM page's worked KV-size example."""
import json
import os

import numpy as np

import workloads
from oracle import kv_bytes

GOLD = os.path.join(os.path.dirname(__file__), "golden", "kv_size_llama2_70b.json")


def test_page_example_is_ten_gib():
    g = json.load(open(GOLD))
    b = kv_bytes.kv_cache_bytes(g["num_layers"], g["num_heads"], g["head_dim"], g["seq_len"],
                                g["bytes_per_elem"])
    assert b == 10_737_418_240 == 10 * 2**30
    # the page rounds it to about 10 GB per request and about 100 GB for 10 requests,
    # more than one 80 GB GPU holds
    assert abs(b / 1e9 - g["page_result_gb_approx"]) / g["page_result_gb_approx"] < 0.08
    assert g["page_requests"] * b / 1e9 > g["page_gpu_capacity_gb"]
    assert abs(g["page_requests"] * b / 1e9 - g["page_total_gb_approx_for_requests"]) < 8


def test_llama2_70b_layer_workload_bytes():
    """The MHA layer workload is one of the page example's 80 layers, 8 requests of 4096 tokens."""
    g = json.load(open(GOLD))
    per_request_layer = kv_bytes.kv_cache_bytes(1, g["num_heads"], g["head_dim"], g["seq_len"], 2)
    c = workloads.CONFIGS[4]
    lens = np.asarray(c.fixed_lens)
    got = kv_bytes.decode_kv_bytes_logical(lens, c.num_kv_heads, c.head_dim, 2)
    assert got == 8 * per_request_layer == 1_073_741_824


def test_unique_bytes_count_shared_blocks_once():
    # two sequences of 40 tokens, bs 16, sharing their first two (full) blocks
    tables = np.array([[7, 3, 1], [7, 3, 2]])
    lens = np.array([40, 40])
    logical = kv_bytes.decode_kv_bytes_logical(lens, 1, 8, 2)
    unique = kv_bytes.decode_kv_bytes_unique(tables, lens, 16, 1, 8, 2)
    assert logical == 2 * 40 * 2 * 8 * 2
    assert unique == (32 + 8 + 8) * 2 * 8 * 2

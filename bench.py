"""Benchmark of the paged decode hot path on one MI355X.

A step is one pass of the whole path over one batch: for every layer of the
workload, kv_append of this step's token per sequence, then paged decode
attention over every sequence's context (plus the merge pass when the plan
splits contexts).  Inputs are seeded synthetic data already resident in HBM.

Default workload: the Llama-3.2-1B-shaped decode batch -- 64 sequences, 32 q /
8 kv heads, head_dim 64, bf16, block size 16, context lengths uniform in
[128, 2048].  To keep the 256 MB last-level cache from serving the KV reads,
the step rotates through R independent copies of the pool, q and outputs
(R * pool bytes >= 1 GiB).

Prints one JSON line on stdout; human-readable details go to stderr.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV GB/s (% of MI355X HBM peak) + decode tokens/s"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s (decimal)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, lens, tables, block_size):
    """Bytes one decode launch must move at minimum, one layer: every context
    token's K and V once per kv head, q in, out back, the table entries read and
    the lengths.  With shared prefix blocks, 'unique' counts each physical slot once."""
    e = cfg.elem_bytes
    per_tok = 2 * cfg.num_kv_heads * cfg.head_dim * e
    nblk = (lens.astype(np.int64) + block_size - 1) // block_size
    small = 2 * len(lens) * cfg.num_q_heads * cfg.head_dim * e + 4 * int(nblk.sum()) + 4 * len(lens)
    logical = int(lens.astype(np.int64).sum()) * per_tok + small
    # unique slots: full blocks once per physical block, partial last blocks per sequence
    uniq_tokens = 0
    full = set()
    for i, L in enumerate(lens):
        for j in range(int(nblk[i])):
            used = min(block_size, int(L) - j * block_size)
            n = int(tables[i, j])
            if used == block_size:
                if n not in full:
                    full.add(n)
                    uniq_tokens += block_size
            else:
                uniq_tokens += used
    unique = uniq_tokens * per_tok + small
    return logical, unique


def append_bytes(cfg, num_tokens):
    return 2 * 2 * num_tokens * cfg.num_kv_heads * cfg.head_dim * cfg.elem_bytes + 8 * num_tokens


def cpu_baseline(wl, budget_s=10.0):
    """The oracle, as it stands, timed on this host over whole passes of the
    workload's first layer until about budget_s seconds have been spent."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        blas = 1
    c, ly = wl.cfg, wl.layers[0]
    kc, vc = ly.k_cache.copy(), ly.v_cache.copy()
    oracle.kv_append(ly.k_new, ly.v_new, wl.slot_mapping, kc, vc, num_blocks=wl.num_blocks, block_size=c.block_size)
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.decode(ly.q, kc, vc, wl.block_tables, wl.context_lens, c.scale, dtype=c.dtype,
                      num_blocks=wl.num_blocks, num_kv_heads=c.num_kv_heads, block_size=c.block_size)
        runs += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / runs
    return dt, runs, blas


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload number (1-5); 2 is the headline")
    ap.add_argument("--impl", default="auto", choices=["auto", "simt", "mfma"])
    ap.add_argument("--partition", type=int, default=0, help="tokens per partition (0 = automatic)")
    ap.add_argument("--rotations", type=int, default=0, help="pool copies to rotate through (0 = enough for 1 GiB)")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle timing (0 = skip)")
    ap.add_argument("--eager", action="store_true", help="launch from Python each step instead of HIP graphs")
    ap.add_argument("--dec-per-graph", type=int, default=8, help="decode calls per captured decode graph")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the decode path has no multi-GPU mode in this build "
              "(see DESIGN.md for how it would shard); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_448_amd as pkv
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    wl = workloads.build(args.config, poison=False)
    c = wl.cfg
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[c.dtype]
    log(f"workload {c.name}: {len(wl.context_lens)} seqs, {c.num_layers} layers, N={wl.num_blocks} blocks, "
        f"generated in {time.time() - t0:.1f}s")

    def up(a, shape=None):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt)
        return (t.reshape(shape) if shape else t).to(dev)

    shape = (wl.num_blocks, c.num_kv_heads, c.block_size // 16, 16 * c.head_dim)
    pool_bytes = 2 * int(np.prod(shape)) * c.elem_bytes * c.num_layers
    R = args.rotations or (1 if c.num_layers > 1 else max(1, math.ceil((1 << 30) / pool_bytes)))
    layers = []  # [rotation][layer] -> dict of device tensors
    for r in range(R):
        rl = []
        for ly in wl.layers:
            rl.append(dict(q=up(ly.q), kc=up(ly.k_cache, shape), vc=up(ly.v_cache, shape), kn=up(ly.k_new),
                           vn=up(ly.v_new), out=torch.empty((len(wl.context_lens), c.num_q_heads, c.head_dim),
                                                             dtype=tdt, device=dev)))
        layers.append(rl)
    tables = torch.from_numpy(wl.block_tables).to(dev)
    lens = torch.from_numpy(wl.context_lens).to(dev)
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    B = len(wl.context_lens)
    mcl = int(wl.context_lens.max())
    ws_bytes = pkv.decode_workspace_bytes(B, c.num_q_heads, c.num_kv_heads, c.head_dim, c.block_size, mcl,
                                          args.partition)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    part = args.partition or pkv.plan_partition(B, c.num_kv_heads, c.block_size, mcl)
    log(f"rotations R={R} ({R * pool_bytes / 2**30:.2f} GiB of pools), partition plan {part or 'single pass'} tokens, "
        f"workspace {ws_bytes} B, impl {args.impl}")

    def decode(t):
        pkv.paged_attn_decode(t["q"], t["kc"], t["vc"], tables, lens, c.scale, t["out"], max_context_len=mcl,
                              workspace=ws, partition_tokens=args.partition, impl=args.impl)

    def step(i):
        for t in layers[i % R]:
            pkv.kv_append(t["kn"], t["vn"], slots, t["kc"], t["vc"])
            decode(t)

    stream = torch.cuda.current_stream(dev)  # the library launches on the current stream
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s = torch.cuda.current_stream(dev)
        e0.record(s)
        for i in range(n):
            fn(i)
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    eager_ms = timed(step, args.steps)

    # The same work replayed from HIP graphs (one per rotation), which removes
    # the Python binding's per-call host time from the GPU's critical path.
    # Inside capture the library launches on the capture stream.
    gstep, gdec = [], []
    if not args.eager:
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(r)
            gstep.append(g)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(args.dec_per_graph):
                    decode(layers[r][0])
            gdec.append(g)
        for r in range(R):
            gstep[r].replay()
            gdec[r].replay()
        torch.cuda.synchronize()
        ms_step = timed(lambda i: gstep[i % R].replay(), args.steps)
        dec_us = 1e3 * timed(lambda i: gdec[i % R].replay(), args.steps) / args.dec_per_graph
    else:
        ms_step = eager_ms
        dec_us = 1e3 * timed(lambda i: decode(layers[i % R][0]), args.steps)
    log(f"eager step {eager_ms * 1e3:.1f} us, {'graph' if not args.eager else 'eager'} step {ms_step * 1e3:.1f} us")

    logical, unique = algorithmic_bytes(c, wl.context_lens, wl.block_tables, c.block_size)
    app = append_bytes(c, B)
    step_bytes = c.num_layers * (unique + app)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    dec_gbs = unique / (dec_us * 1e-6) / 1e9
    log(f"step {ms_step * 1e3:.1f} us ({c.num_layers} layers), decode call {dec_us:.1f} us "
        f"; decode bytes {unique / 1e6:.2f} MB unique, "
        f"{logical / 1e6:.2f} MB logical -> {dec_gbs:.0f} GB/s = {100 * dec_gbs / HBM_PEAK_GBS:.1f}% of peak")

    cpu = None
    if args.cpu_budget > 0:
        dt, runs, blas = cpu_baseline(wl, args.cpu_budget)
        cpu = {"value": round(unique / dt / 1e9, 4), "unit": "GB/s", "cores": blas, "kind": "oracle",
               "sample": f"whole first layer of the workload ({B} sequences), {runs} oracle passes, "
                         f"{dt:.3f} s per pass; numpy fp64 with {blas} BLAS thread(s) on "
                         f"{len(os.sched_getaffinity(0))} available host cores",
               "tokens_per_s": round(B / dt, 2)}
        log(f"cpu oracle: {dt:.3f} s per pass over {B} sequences ({runs} passes)")

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic",
        "config": {"workload": f"{c.name}: decode step (kv_append + paged decode) of {B} sequences, "
                               f"{c.num_layers} layer(s), {c.num_q_heads}q/{c.num_kv_heads}kv heads, "
                               f"head_dim {c.head_dim}, block_size {c.block_size}",
                   "config_id": args.config, "num_seqs": B, "num_layers": c.num_layers,
                   "num_q_heads": c.num_q_heads, "num_kv_heads": c.num_kv_heads, "head_dim": c.head_dim,
                   "block_size": c.block_size, "context_tokens": int(wl.context_lens.sum()),
                   "max_context_len": mcl, "seed": wl.seed, "impl": args.impl, "partition_tokens": part,
                   "rotations": R},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "decode_call_us": round(dec_us, 2),
        "decode_bytes_unique": unique,
        "decode_bytes_logical": logical,
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "paged_attn_decode call (partition kernel + merge pass when split)"},
        "launch": "eager" if args.eager else "hip-graph",
        "eager_ms_per_step": round(eager_ms, 5),
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the paged decode hot path on one MI355X.

A step is one pass of the whole path over one batch: for every layer of the
workload, kv_append of this step's token per sequence, then paged decode
attention over every sequence's context (plus the merge pass when the plan
splits contexts).  By default each layer is one append_paged_attn_decode
launch (append fused into the decode kernel); --unfused times the two calls.
Inputs are seeded synthetic data already resident in HBM.

Default workload: the Llama-3.2-1B-shaped decode batch -- 64 sequences, 32 q /
8 kv heads, head_dim 64, bf16, block size 16, context lengths uniform in
[128, 2048].  So that the 256 MB last-level cache cannot serve the KV reads,
step i uses copy i mod R of the pools, q and outputs, with R copies adding up
to at least 1 GiB (one-layer workloads; the 16-layer workload is cold by
itself).

Timing: W warm-up steps, then exactly K steps between two device
synchronisations, enqueued behind a device-side sleep so that the GPU runs
them back to back; timing events recorded on the stream the kernels run on
bracket the K steps.  Fused, a step is one launch per layer, so the per-launch
duration is the bracketed time over K x layers launches (inter-kernel gaps
included).  Unfused, events also bracket each decode call (an event between
two kernels adds idle time, so that figure errs high).

Prints one JSON line on stdout; human-readable details go to stderr.

Other modes (measurement tooling):
  --copy-calibration  after the timed steps, run a plain device copy of a
                      known size three times, so that a rocprofv3 --pmc run of
                      this command also reads the counters of a kernel whose
                      HBM bytes are known.
  --pmc-summary FETCH_CSV WRITE_CSV
                      turn the counter_collection.csv files of two such runs
                      (FETCH_SIZE, then WRITE_SIZE) into the traffic summary
                      under profiles/ that later runs report as
                      roofline.traffic while the decode sources are unchanged.
  --kv fp8            the step over FP8 (E4M3) pools: kv_append_fp8 + paged
                      decode over the quantised pools; its own JSON line.
  --prefill           paged prefill: every context of the workload is a prompt
                      whose tokens are all new; reports TFLOP/s of the causal
                      attention against the dense MFMA peak; its own JSON line.
  --loop NAME         continuous-batching loop instead of one batch: requests
                      are admitted (prompt K/V written), decode one token per
                      step over all layers, and leave, for W + K steps of a
                      seeded plan (workloads.loop); reports sustained decode
                      tokens/s over the K timed steps, host scheduling, copies
                      and prompt writes included.  Its own JSON line.
"""
import argparse
import hashlib
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
CSRC = os.path.join(ROOT, "paged_kv_cache_448_amd", "csrc")
# sources whose change invalidates measured counters of the decode kernels
DECODE_SOURCES = ["common.h", "kernels.h", "decode_common.h", "decode_mfma_kernel.h", "decode_mfma.hip",
                  "decode_fp8.hip", "decode_simt.hip", "merge.hip", "api.cpp"]
COPY_CALIBRATION_BYTES = 1 << 29  # 512 MiB read and written by the calibration copy


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_sources_sha():
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_summary_path(workload_name):
    return os.path.join(ROOT, "profiles", f"decode_traffic_{workload_name}.txt")


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


def per_layer_read(wl, plan, cfg):
    """Pool bytes the prefix decode reads per layer: each prefix item's shared
    blocks once, every sequence's own positions after its prefix."""
    per_tok = 2 * cfg.num_kv_heads * cfg.head_dim * cfg.elem_bytes
    return per_tok * (sum(int(plan.prefix_len[it[0]]) for it in plan.items) +
                      int((wl.context_lens.astype(np.int64) - plan.prefix_len).sum()))


def append_bytes(cfg, num_tokens):
    return 2 * 2 * num_tokens * cfg.num_kv_heads * cfg.head_dim * cfg.elem_bytes + 8 * num_tokens


def _blas_threads():
    """Threads the oracle's numpy BLAS runs with (its matrix products are its only parallel part)."""
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        return 1


def cpu_baseline(wl, budget_s=10.0):
    """The oracle, as it stands, timed on this host over whole passes of the
    workload's first layer until about budget_s seconds have been spent."""
    import oracle
    blas = _blas_threads()
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


def _read_counter_csv(path, counter):
    """(kernel name, grid size, value) per dispatch for one counter of a rocprofv3 counter_collection.csv."""
    import csv
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                rows.append((r.get("Kernel_Name", ""), int(r.get("Grid_Size", 0)), float(r["Counter_Value"])))
    return rows


def pmc_summary(fetch_csv, write_csv, workload_name, decode_bytes, steps_note,
                kernels=("decode_mfma_kernel", "decode_simt_kernel")):
    """Traffic per decode launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for the calibration copy."""
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _read_counter_csv(path, counter)
        # the timed launches: with the fused append the grid carries extra append
        # workgroups, which tells them from the decode-only context loop
        dec_rows = [(g, v) for n, g, v in rows if any(k in n for k in kernels)]
        top = max((g for g, _ in dec_rows), default=0)
        dec = [v for g, v in dec_rows if g == top]
        mrg = [v for n, g, v in rows if "merge_kernel" in n]
        # the calibration copies are the three largest copy dispatches
        cpy = sorted(v for n, g, v in rows if "copy" in n.lower())[-3:]
        if not dec or not cpy:
            raise SystemExit(f"{path}: no decode ({len(dec)}) or copy ({len(cpy)}) dispatches with {counter}")
        copy_kib = float(np.median(cpy))
        factor = COPY_CALIBRATION_BYTES / (copy_kib * 1024.0)
        dec_kib = float(np.mean(dec)) + (float(np.mean(mrg)) if mrg else 0.0)
        out[counter] = {"decode_kib_per_launch": dec_kib, "decode_dispatches": len(dec),
                        "merge_kib_per_launch": float(np.mean(mrg)) if mrg else 0.0,
                        "copy_kib_per_dispatch": copy_kib, "copy_bytes": COPY_CALIBRATION_BYTES,
                        "scale_factor": factor, "bytes_per_launch": dec_kib * 1024.0 * factor}
    rec = {"workload": workload_name, "decode_sources_sha": decode_sources_sha(),
           "traffic_bytes_per_launch": out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"],
           "algorithmic_bytes_per_launch": decode_bytes, "counters": out, "run": steps_note}
    path = traffic_summary_path(workload_name)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    log(f"wrote {path}: traffic {rec['traffic_bytes_per_launch'] / 1e6:.1f} MB per launch vs "
        f"{decode_bytes / 1e6:.1f} MB algorithmic")
    return rec


def load_traffic(workload_name):
    path = traffic_summary_path(workload_name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("decode_sources_sha") != decode_sources_sha():
        log(f"{path} was measured on other decode sources; traffic not reported")
        return None
    return rec["traffic_bytes_per_launch"]


def loop_bench(name, steps, warmup, seed=11, schedule=True):
    """Sustained decode tokens/s of the continuous-batching loop (see --loop)."""
    import torch

    from paged_kv_cache_448_amd.loop import DecodeLoop
    from workloads import loop as wl_loop

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lc = wl_loop.LOOP_CONFIGS[name]
    reqs, plan = wl_loop.plan(lc, seed, warmup + steps)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    most_prompt = max(sum(reqs[r].prompt_len for r in st.admit) for st in plan)
    loop = DecodeLoop(lc, dev, max_prompt_tokens=most_prompt, schedule=schedule)
    tdt = loop.dtype
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    B = lc.max_batch
    # values do not change the work, so every step reuses one set of them
    q = torch.randn((B, lc.num_q_heads, lc.head_dim), generator=g, device=dev).to(tdt)
    kn = torch.randn((B, lc.num_kv_heads, lc.head_dim), generator=g, device=dev).to(tdt)
    vn = torch.randn((B, lc.num_kv_heads, lc.head_dim), generator=g, device=dev).to(tdt)
    kp = torch.randn((most_prompt, lc.num_kv_heads, lc.head_dim), generator=g, device=dev).to(tdt)
    vp = torch.randn((most_prompt, lc.num_kv_heads, lc.head_dim), generator=g, device=dev).to(tdt)
    outs = [torch.empty((B, lc.num_q_heads, lc.head_dim), dtype=tdt, device=dev) for _ in range(lc.num_layers)]
    per_token_kv = 2 * lc.num_kv_heads * lc.head_dim * 2

    def run(st):
        if st.admit:
            lens_p = [reqs[rid].prompt_len for rid in st.admit]
            T = sum(lens_p)
            loop.admit(st.admit, lens_p, lambda layer, cached: (kp[:T], vp[:T]))
        n = len(st.run)
        lens = loop.decode_step(st.run, lambda layer: (q[:n], kn[:n], vn[:n]), [o[:n] for o in outs])
        for rid in st.finish:
            loop.finish(rid)
        return n, int(np.asarray(lens, dtype=np.int64).sum()), sum(reqs[r].prompt_len for r in st.admit)

    for st in plan[:warmup]:
        run(st)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    tokens = ctx_tokens = prompt_tokens = 0
    loop.host_wait_s = 0.0
    h0 = time.perf_counter()
    e0.record(stream)
    for st in plan[warmup:]:
        n, c, pt = run(st)
        tokens += n
        ctx_tokens += c
        prompt_tokens += pt
    e1.record(stream)
    host_s = time.perf_counter() - h0
    torch.cuda.synchronize()
    gpu_ms = e0.elapsed_time(e1)
    wall_s = max(gpu_ms / 1e3, host_s)
    kv_bytes = ctx_tokens * per_token_kv * lc.num_layers
    log(f"loop {name}: {steps} steps, {tokens} decode tokens (batch {tokens / steps:.1f} on average), "
        f"{prompt_tokens} prompt tokens written; GPU {gpu_ms:.2f} ms, host enqueue {host_s * 1e3:.2f} ms "
        f"(of which {loop.host_wait_s * 1e3:.2f} ms waiting for the GPU); "
        f"{kv_bytes / 1e9:.2f} GB of context K/V read")
    rec = {"metric": "continuous-batching decode tokens/s", "value": round(tokens / wall_s, 1), "unit": "tokens/s",
           "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(wall_s * 1e3 / steps, 4),
           "higher_is_better": True, "dtype": lc.dtype, "data": "synthetic",
           "config": {"workload": f"{name}: {lc.num_layers} layers, {lc.num_q_heads}q/{lc.num_kv_heads}kv heads, "
                                  f"head_dim {lc.head_dim}, block_size {lc.block_size}, batch up to {lc.max_batch}, "
                                  f"seed {seed}"},
           "avg_batch": round(tokens / steps, 2), "gpu_ms": round(gpu_ms, 3), "host_enqueue_ms": round(host_s * 1e3, 3),
           "host_wait_ms": round(loop.host_wait_s * 1e3, 3),
           "kv_read_gbs": round(kv_bytes / (wall_s * 1e9), 1),
           "kv_read_frac_of_peak": round(kv_bytes / (wall_s * 1e9) / HBM_PEAK_GBS, 4),
           "schedule": "host dispatch order (pkv_decode_schedule)" if schedule else "sequence order"}
    print(json.dumps(rec), flush=True)


def prefill_flops(lens, new, num_q_heads, head_dim):
    """Matrix-core flops of causal prefill: each new token at position p scores and
    accumulates over p + 1 keys, 2*D flops each for q.K and for P.V, per q head."""
    total = 0
    for L, n in zip(lens, new):
        L, n = int(L), int(n)
        # sum over positions p = L-n .. L-1 of (p + 1)
        total += n * (2 * L - n + 1) // 2
    return 4 * head_dim * num_q_heads * total


def prefill_bench(config, steps, warmup, cpu_budget):
    """Paged prefill of whole prompts (see --prefill): every context of the workload is a
    prompt whose tokens are all new."""
    import torch

    import paged_kv_cache_448_amd as pkv
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.build(config, poison=False)
    c = wl.cfg
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[c.dtype]
    lens = wl.context_lens
    new = [int(x) for x in lens]
    B, T = len(new), int(sum(new))
    rng = np.random.default_rng(5)
    q_bits = workloads.random_bits(rng, (T, c.num_q_heads, c.head_dim), c.dtype)

    def up(a, shape=None):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt)
        return (t.reshape(shape) if shape else t).to(dev)

    shape = (wl.num_blocks, c.num_kv_heads, c.block_size, c.head_dim)
    ly = wl.layers[0]
    q = up(q_bits)
    kc, vc = up(ly.k_cache, shape), up(ly.v_cache, shape)
    out = torch.empty_like(q)
    tables = torch.from_numpy(wl.block_tables).to(dev)
    lens_d = torch.from_numpy(lens).to(dev)
    qs = torch.from_numpy(np.concatenate([[0], np.cumsum(new)]).astype(np.int32)).to(dev)
    mql, mcl = max(new), int(lens.max())

    def call(i):
        pkv.paged_prefill(q, kc, vc, tables, lens_d, qs, c.scale, out, max_query_len=mql, max_context_len=mcl)

    stream = torch.cuda.current_stream(dev)
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        call(i)
    b.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * a.elapsed_time(b) / steps
    flops = prefill_flops(lens, new, c.num_q_heads, c.head_dim)
    tfs = flops / (us * 1e-6) / 1e12
    peak = 2500.0  # MI355X dense bf16 / fp16 MFMA, TFLOP/s
    log(f"prefill {c.name}: {B} prompts, {T} tokens, {flops / 1e9:.1f} GFLOP per call; {us:.1f} us per call -> "
        f"{tfs:.1f} TFLOP/s = {100 * tfs / peak:.1f}% of the dense MFMA peak")
    cpu = None
    if cpu_budget > 0:
        from oracle.prefill import prefill as oracle_prefill
        # sample: the shortest prompts, whole, until the budget is spent
        order = np.argsort(lens)
        done_flops, t0, used = 0, time.perf_counter(), []
        for i in order:
            sub_qs = np.array([0, new[i]])
            s0 = int(np.concatenate([[0], np.cumsum(new)])[i])
            oracle_prefill(q_bits[s0:s0 + new[i]], ly.k_cache, ly.v_cache, wl.block_tables[i:i + 1], lens[i:i + 1],
                           sub_qs, c.scale, dtype=c.dtype, num_blocks=wl.num_blocks, num_kv_heads=c.num_kv_heads,
                           block_size=c.block_size)
            done_flops += prefill_flops(lens[i:i + 1], new[i:i + 1], c.num_q_heads, c.head_dim)
            used.append(int(new[i]))
            if time.perf_counter() - t0 >= cpu_budget:
                break
        dt = time.perf_counter() - t0
        cpu = {"value": round(done_flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
               "sample": f"oracle.prefill over {len(used)} whole prompts of the batch ({sum(used)} tokens, "
                         f"the shortest first), {dt:.1f} s"}
    rec = {"metric": "paged prefill attention TFLOP/s (% of MI355X dense MFMA peak)", "value": round(tfs, 2),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(us / 1e3, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": c.dtype, "data": "synthetic",
           "config": {"workload": f"{c.name} contexts as whole prompts: paged_prefill of {B} prompts, {T} tokens, "
                                  f"{c.num_q_heads}q/{c.num_kv_heads}kv heads, head_dim {c.head_dim}, "
                                  f"block_size {c.block_size}", "config_id": config, "flops_per_call": flops},
           "prefill_tokens_per_s": round(T / (us * 1e-6), 1),
           "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": peak, "unit": "TFLOP/s",
                        "frac": round(tfs / peak, 4), "traffic": None, "kernel": "prefill_mfma_kernel"},
           "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


def fp8_decode_bytes(wl):
    """Algorithmic bytes of one decode launch over FP8 pools: the unique context
    K/V at one byte per element, plus q, out, table entries and lengths."""
    c = wl.cfg
    B, bs = len(wl.context_lens), c.block_size
    _, unique16 = algorithmic_bytes(c, wl.context_lens, wl.block_tables, bs)
    small = 2 * B * c.num_q_heads * c.head_dim * c.elem_bytes + 4 * int(((wl.context_lens + bs - 1) // bs).sum()) + 4 * B
    return (unique16 - small) // c.elem_bytes + small


def fp8_bench(config, steps, warmup, cpu_budget, copy_calibration=False, k_scale=0.0125, v_scale=0.01,
              schedule="host", fused=True):
    """Decode step over FP8 (E4M3) pools (see --kv fp8): per layer, the append of this
    step's token per sequence and paged_attn_decode_fp8, as one launch
    (append_paged_attn_decode_fp8) or, unfused, kv_append_fp8 and the decode."""
    import torch

    import paged_kv_cache_448_amd as pkv
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.build(config, poison=False)
    c = wl.cfg
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[c.dtype]
    N, Hkv, bs, D = wl.num_blocks, c.num_kv_heads, c.block_size, c.head_dim
    B = len(wl.context_lens)

    def up(a, shape=None):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt)
        return (t.reshape(shape) if shape else t).to(dev)

    all_slots = torch.arange(N * bs, dtype=torch.int64, device=dev)

    def fp8_pools(k_bits, v_bits):
        # every slot of the 16-bit pools, quantised by the library's own append
        def rows(bits):
            return up(bits, (N, Hkv, bs, D)).permute(0, 2, 1, 3).reshape(N * bs, Hkv, D).contiguous()
        kp, vp = pkv.new_cache_fp8(N, Hkv, bs, D, dev), pkv.new_cache_fp8(N, Hkv, bs, D, dev)
        pkv.kv_append_fp8(rows(k_bits), rows(v_bits), all_slots, kp, vp, k_scale, v_scale)
        return kp, vp

    pool_bytes = 2 * N * Hkv * bs * D * c.num_layers
    R = 1 if c.num_layers > 1 else max(1, math.ceil((1 << 30) / pool_bytes))
    layers = []
    for r in range(R):
        rl = []
        for ly in wl.layers:
            kp, vp = fp8_pools(ly.k_cache, ly.v_cache)
            rl.append(dict(q=up(ly.q), kc=kp, vc=vp, kn=up(ly.k_new), vn=up(ly.v_new),
                           out=torch.empty((B, c.num_q_heads, D), dtype=tdt, device=dev)))
        layers.append(rl)
    torch.cuda.synchronize()
    tables = torch.from_numpy(wl.block_tables).to(dev)
    lens = torch.from_numpy(wl.context_lens).to(dev)
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    order = torch.from_numpy(pkv.decode_schedule(wl.context_lens)).to(dev) if schedule == "host" else None
    mcl = int(wl.context_lens.max())
    ws = torch.empty(max(pkv.decode_workspace_bytes(B, c.num_q_heads, Hkv, D, bs, mcl), 256), dtype=torch.uint8,
                     device=dev)
    part = pkv.plan_partition(B, Hkv, bs, mcl)
    log(f"fp8 kv: workload {c.name}, rotations R={R} ({R * pool_bytes / 2**30:.2f} GiB of pools), "
        f"partition plan {part or 'single pass'}")

    def decode(t):
        pkv.paged_attn_decode_fp8(t["q"], t["kc"], t["vc"], tables, lens, c.scale, k_scale, v_scale, t["out"],
                                  max_context_len=mcl, workspace=ws, seq_order=order)

    def step(i):
        for t in layers[i % R]:
            if fused:
                pkv.append_paged_attn_decode_fp8(t["q"], t["kn"], t["vn"], slots, t["kc"], t["vc"], tables, lens,
                                                 c.scale, k_scale, v_scale, t["out"], max_context_len=mcl,
                                                 workspace=ws, seq_order=order)
                continue
            pkv.kv_append_fp8(t["kn"], t["vn"], slots, t["kc"], t["vc"], k_scale, v_scale)
            decode(t)

    stream = torch.cuda.current_stream(dev)
    h0 = time.perf_counter()
    for i in range(warmup):
        step(i)
    host_per_step = (time.perf_counter() - h0) / max(warmup, 1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    torch.cuda._sleep(1 << 20)
    e1.record(stream)
    torch.cuda.synchronize()
    cycles_per_us = (1 << 20) / max(1e3 * e0.elapsed_time(e1), 1e-3)
    head_us = max(2000.0, 1.5e6 * host_per_step * steps)

    def timed(fn):
        torch.cuda.synchronize()
        torch.cuda._sleep(int(head_us * cycles_per_us))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(steps):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    ms_step = timed(step) / steps
    dec_us = 1e3 * timed(lambda i: [decode(t) for t in layers[i % R]]) / (steps * c.num_layers)

    if copy_calibration:
        src = torch.empty(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    unique = fp8_decode_bytes(wl)
    app = 2 * B * Hkv * D * (c.elem_bytes + 1) + 8 * B
    value = c.num_layers * (unique + app) / (ms_step * 1e-3) / 1e9
    dec_gbs = unique / (dec_us * 1e-6) / 1e9
    # fused, a step is one launch per layer: the roofline is that launch's (as for 16-bit pools)
    launch_us = 1e3 * ms_step / c.num_layers if fused else dec_us
    launch_bytes = unique + app if fused else unique
    launch_gbs = launch_bytes / (launch_us * 1e-6) / 1e9
    log(f"fp8 step {ms_step * 1e3:.1f} us; decode call {dec_us:.2f} us over {unique / 1e6:.2f} MB -> {dec_gbs:.0f} GB/s "
        f"= {100 * dec_gbs / HBM_PEAK_GBS:.1f}% of peak")
    cpu = None
    if cpu_budget > 0:
        from oracle import fp8 as ofp8
        ly = wl.layers[0]
        # the oracle's append of the contexts is the sample's setup, not timed
        rows = lambda bits: bits.reshape(N, Hkv, bs, D).transpose(0, 2, 1, 3).reshape(N * bs, Hkv, D)  # noqa: E731
        kc = np.full((N, Hkv, bs, D), ofp8.NAN_CODE, np.uint8)
        vc = np.full_like(kc, ofp8.NAN_CODE)
        ctx = np.unique(np.concatenate([wl.block_tables[i, np.arange(int(L)) // bs].astype(np.int64) * bs
                                        + np.arange(int(L)) % bs for i, L in enumerate(wl.context_lens)]))
        ofp8.append(rows(ly.k_cache)[ctx], rows(ly.v_cache)[ctx], c.dtype, ctx, kc, vc, k_scale, v_scale,
                    num_blocks=N, block_size=bs)
        runs, t0 = 0, time.perf_counter()
        while True:
            ofp8.decode(ly.q, kc, vc, k_scale, v_scale, wl.block_tables, wl.context_lens, c.scale, q_dtype=c.dtype,
                        num_blocks=N, num_kv_heads=Hkv, block_size=bs)
            runs += 1
            if time.perf_counter() - t0 >= cpu_budget:
                break
        dt = (time.perf_counter() - t0) / runs
        cpu = {"value": round(unique / dt / 1e9, 4), "unit": "GB/s", "cores": _blas_threads(), "kind": "oracle",
               "sample": f"oracle.fp8.decode over the whole first layer ({B} sequences), {runs} passes, "
                         f"{dt:.3f} s per pass", "tokens_per_s": round(B / dt, 2)}
    traffic = load_traffic(c.name + "-fp8")
    if traffic is not None:
        traffic = int(round(traffic))
    rec = {"metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
           "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": f"kv fp8-e4m3, q/out/mfma {c.dtype}", "data": "synthetic",
           "config": {"workload": f"{c.name} over FP8 (E4M3) pools: FP8 append + paged_attn_decode_fp8 of {B} "
                                  f"sequences, {c.num_layers} layer(s), {c.num_q_heads}q/{Hkv}kv heads, head_dim {D}, "
                                  f"block_size {bs}", "config_id": config, "kv": "fp8_e4m3",
                      "k_scale": k_scale, "v_scale": v_scale, "partition_tokens": part, "rotations": R},
           "schedule": ("host dispatch order (pkv_decode_schedule)" if order is not None else "sequence order"),
           "append": "fused into the decode kernel" if fused else "separate kv_append_fp8 kernel",
           "decode_tokens_per_s": round(B / (ms_step * 1e-3), 1), "decode_call_us": round(launch_us, 2),
           "decode_bytes_unique": unique,
           "roofline": {"bound": "hbm", "achieved": round(launch_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(launch_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                        "kernel": ("decode_fp8_kernel with the FP8 append fused, one launch per layer" if fused
                                   else "decode_fp8_kernel (paged_attn_decode_fp8 call)")},
           "launch_bytes": launch_bytes, "decode_only_call_us": round(dec_us, 2),
           "decode_only_hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
           "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


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
    ap.add_argument("--copy-calibration", action="store_true", help="also run a plain copy of known size")
    ap.add_argument("--unfused", action="store_true", help="time kv_append and paged_attn_decode as two calls")
    ap.add_argument("--graph", action="store_true",
                    help="capture the K timed steps into one HIP graph and replay it (fused path only)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--loop", default=None, help="continuous-batching loop workload (e.g. cb-llama3.2-1b)")
    ap.add_argument("--prefill", action="store_true",
                    help="paged prefill of the workload's contexts as whole prompts (TFLOP/s)")
    ap.add_argument("--schedule", default="host", choices=["host", "none"],
                    help="host: pass the dispatch order pkv_decode_schedule makes from the lengths; none: sequence order")
    ap.add_argument("--prefix", default="auto", choices=["auto", "off"],
                    help="read prefix blocks shared by several sequences once per prefix item "
                         "(auto: when the host's block tables share any; off: every sequence reads its own)")
    ap.add_argument("--work-list", default="auto", choices=["auto", "on", "off"],
                    help="launch only the partitions that hold tokens (a host work list, "
                         "pkv_decode_work_list) when the plan splits contexts: auto with prefix items, on always, "
                         "off never (the full grid)")
    ap.add_argument("--kv", default="16bit", choices=["16bit", "fp8"],
                    help="fp8: the step over FP8 (E4M3) pools (append + paged_attn_decode_fp8, fused unless --unfused)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the decode path has no multi-GPU mode (each GPU would run "
              "its own sequences or kv heads on its own pools); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.loop:
        loop_bench(args.loop, args.steps, args.warmup, schedule=args.schedule == "host")
        return
    if args.prefill:
        prefill_bench(args.config, args.steps, args.warmup, args.cpu_budget)
        return
    if args.kv == "fp8" and not args.pmc_summary:
        fp8_bench(args.config, args.steps, args.warmup, args.cpu_budget, args.copy_calibration,
                  schedule=args.schedule, fused=not args.unfused)
        return

    import workloads
    if args.pmc_summary:
        wl = workloads.build(args.config, poison=False)
        B, c = len(wl.context_lens), wl.cfg
        if args.kv == "fp8":
            # the counter runs time the fused step: its launch also reads the appended
            # tokens' 16-bit K/V and writes their codes
            app8 = 2 * B * c.num_kv_heads * c.head_dim * (c.elem_bytes + 1) + 8 * B
            pmc_summary(args.pmc_summary[0], args.pmc_summary[1], wl.cfg.name + "-fp8", fp8_decode_bytes(wl) + app8,
                        f"bench.py --kv fp8 --config {args.config} --steps {args.steps} --warmup {args.warmup} "
                        f"--cpu-budget 0 --copy-calibration", kernels=("decode_fp8_kernel",))
            return
        _, unique = algorithmic_bytes(wl.cfg, wl.context_lens, wl.block_tables, wl.cfg.block_size)
        # the counter runs time the fused launch (decode + the appended tokens' K/V)
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], wl.cfg.name, unique + append_bytes(c, B),
                    f"bench.py --config {args.config} --steps {args.steps} --warmup {args.warmup} "
                    f"--cpu-budget 0 --copy-calibration")
        return

    import torch

    import paged_kv_cache_448_amd as pkv

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

    shape = (wl.num_blocks, c.num_kv_heads, c.block_size, c.head_dim)
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
    # dispatch order from the host's copy of the lengths (as the block tables)
    order = torch.from_numpy(pkv.decode_schedule(wl.context_lens)).to(dev) if args.schedule == "host" else None
    mcl = int(wl.context_lens.max())
    # shared prefixes, from the host's copy of the tables (as the dispatch order)
    plan = None
    if args.prefix == "auto" and args.impl != "simt" and pkv.decode_supported("mfma", c.dtype, c.head_dim, c.group):
        plan = pkv.decode_prefix_plan(wl.block_tables, wl.context_lens, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                      c.block_size)
        if plan.num_items == 0:
            plan = None
    if plan is not None:
        pre_len = torch.from_numpy(plan.prefix_len).to(dev)
        pre_items = torch.from_numpy(np.ascontiguousarray(plan.items)).to(dev)
        ws_bytes = pkv.decode_prefix_workspace_bytes(B, c.num_q_heads, c.num_kv_heads, c.head_dim, c.block_size, mcl,
                                                     plan.max_prefix_len, args.partition)
        log(f"shared prefixes: {plan.num_items} prefix items, longest prefix {plan.max_prefix_len} tokens, "
            f"{int(plan.prefix_len.sum())} prefix tokens read once per item")
    else:
        ws_bytes = pkv.decode_workspace_bytes(B, c.num_q_heads, c.num_kv_heads, c.head_dim, c.block_size, mcl,
                                              args.partition)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    part = args.partition or pkv.plan_partition(B, c.num_kv_heads, c.block_size, mcl)
    # split plans: the live (sequence, partition) entries, from the host's lengths
    work = None
    # (without prefix items the full grid measured as fast or faster: workload 5 48.1 against
    # 50.0 us per layer, workload 3 within noise)
    want_list = args.work_list == "on" or (args.work_list == "auto" and plan is not None)
    if (want_list and part and args.impl != "simt" and
            pkv.decode_supported("mfma", c.dtype, c.head_dim, c.group)):
        wl_np = pkv.decode_work_list(wl.context_lens, c.num_kv_heads, mcl, args.partition,
                                     None if plan is None else plan.prefix_len)
        work = torch.from_numpy(wl_np).to(dev)
        if plan is None:
            # the prefix entry point with no items is the plain decode; it takes the work list
            plan = pkv.PrefixPlan(np.zeros(B, np.int32), np.zeros((0, 16), np.int32), 0)
            pre_len = torch.zeros(B, dtype=torch.int32, device=dev)
            pre_items = torch.full((1, 16), -1, dtype=torch.int32, device=dev)
        log(f"work list: {len(wl_np)} live (sequence, partition) entries of {B * -(-mcl // part)} in the grid")
    shared = plan is not None and plan.num_items > 0
    log(f"rotations R={R} ({R * pool_bytes / 2**30:.2f} GiB of pools), partition plan {part or 'single pass'} tokens, "
        f"workspace {ws_bytes} B, impl {args.impl}")

    def decode(t):
        if plan is not None:
            pkv.paged_attn_decode_prefix(t["q"], t["kc"], t["vc"], tables, lens, c.scale, pre_len, pre_items,
                                         plan.max_prefix_len, t["out"], max_context_len=mcl, workspace=ws,
                                         partition_tokens=args.partition, seq_order=order, work=work)
            return
        pkv.paged_attn_decode(t["q"], t["kc"], t["vc"], tables, lens, c.scale, t["out"], max_context_len=mcl,
                              workspace=ws, partition_tokens=args.partition, impl=args.impl, seq_order=order)

    fused = not args.unfused
    if fused and not pkv.decode_supported("mfma", c.dtype, c.head_dim, c.group):
        log("the fused append + decode needs the MFMA kernel; timing two calls")
        fused = False
    if fused and args.impl == "simt":
        log("--impl simt: timing two calls (the append is fused into the MFMA kernel only)")
        fused = False

    def step(i, evs=None):
        for li, t in enumerate(layers[i % R]):
            if fused and plan is not None:
                pkv.paged_attn_decode_prefix(t["q"], t["kc"], t["vc"], tables, lens, c.scale, pre_len, pre_items,
                                             plan.max_prefix_len, t["out"], k_new=t["kn"], v_new=t["vn"],
                                             slot_mapping=slots, max_context_len=mcl, workspace=ws,
                                             partition_tokens=args.partition, seq_order=order, work=work)
                continue
            if fused:
                pkv.append_paged_attn_decode(t["q"], t["kn"], t["vn"], slots, t["kc"], t["vc"], tables, lens, c.scale,
                                             t["out"], max_context_len=mcl, workspace=ws,
                                             partition_tokens=args.partition, seq_order=order)
                continue
            pkv.kv_append(t["kn"], t["vn"], slots, t["kc"], t["vc"])
            if evs is not None:
                evs[i][li][0].record()
            decode(t)
            if evs is not None:
                evs[i][li][1].record()

    stream = torch.cuda.current_stream(dev)  # the library launches on the current stream
    t_host = time.perf_counter()
    for i in range(args.warmup):
        step(i)
    host_per_step = (time.perf_counter() - t_host) / max(args.warmup, 1)
    torch.cuda.synchronize()

    # Host-side launches cost about as much time as the GPU work of a step, so
    # the timed steps are enqueued behind a device-side sleep long enough for
    # the host to queue all of them: the GPU then runs them back to back and
    # the events around each decode call bracket only that call's kernels.
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    torch.cuda._sleep(1 << 20)
    e1.record(stream)
    torch.cuda.synchronize()
    cycles_per_us = (1 << 20) / max(1e3 * e0.elapsed_time(e1), 1e-3)
    head_us = max(2000.0, 1.5e6 * host_per_step * K)
    evs = None if fused else [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                               for _ in range(c.num_layers)] for _ in range(K)]
    t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    graph = None
    if args.graph and fused:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(K):
                step(i)
        graph.replay()  # untimed: uploads the graph
        torch.cuda.synchronize()

    # timed region: exactly K steps between two synchronisations
    torch.cuda.synchronize()
    if graph is None:
        torch.cuda._sleep(int(head_us * cycles_per_us))
    t_begin.record(stream)
    t_host = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for i in range(K):
            step(i, evs)
    host_us = 1e6 * (time.perf_counter() - t_host)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_begin.elapsed_time(t_end) / K
    launch = "one HIP graph of the K steps" if graph is not None else "eager, queued ahead of the GPU"
    if graph is None and host_us > head_us + 1e3 * ms_step * K:
        launch = "eager, host-bound (GPU may have idled between steps)"
        log(f"warning: enqueueing took {host_us:.0f} us, more than the {head_us:.0f} us head start plus GPU time")
    if fused:
        dec_us = 1e3 * ms_step / c.num_layers
        log(f"step {ms_step * 1e3:.1f} us ({c.num_layers} layer(s), one fused launch each): {dec_us:.2f} us per "
            f"launch; host enqueue {host_us:.0f} us behind a {head_us:.0f} us head start")
    else:
        dec_us_all = [1e3 * a.elapsed_time(b) for per_step in evs for (a, b) in per_step]
        dec_us = float(np.mean(dec_us_all))
        log(f"step {ms_step * 1e3:.1f} us ({c.num_layers} layer(s)); decode call mean {dec_us:.2f} us, "
            f"median {float(np.median(dec_us_all)):.2f}, min {min(dec_us_all):.2f}, max {max(dec_us_all):.2f} "
            f"over {len(dec_us_all)} calls; host enqueue {host_us:.0f} us behind a {head_us:.0f} us head start")

    # Context, outside the K timed steps: the decode kernel alone (no append),
    # K calls back to back over the rotating copies, events around all of them.
    decode_only_us = None
    if True:
        torch.cuda.synchronize()
        torch.cuda._sleep(int(head_us * cycles_per_us))
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for i in range(K):
            for t in layers[i % R]:
                decode(t)
        d1.record(stream)
        torch.cuda.synchronize()
        decode_only_us = 1e3 * d0.elapsed_time(d1) / (K * c.num_layers)
        log(f"decode kernel alone (separate loop, context): {decode_only_us:.2f} us per call")

    if args.copy_calibration:
        src = torch.empty(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    logical, unique = algorithmic_bytes(c, wl.context_lens, wl.block_tables, c.block_size)
    app = append_bytes(c, B)
    step_bytes = c.num_layers * (unique + app)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    launch_bytes = unique + app if fused else unique  # the fused launch also moves the appended tokens
    dec_gbs = launch_bytes / (dec_us * 1e-6) / 1e9
    log(f"decode bytes {unique / 1e6:.2f} MB unique, {logical / 1e6:.2f} MB logical per layer"
        + ("" if not shared else f" (prefix items: the kernels read {per_layer_read(wl, plan, c) / 1e6:.2f} MB)")
        + "; "
        f"{launch_bytes / 1e6:.2f} MB per launch -> {dec_gbs:.0f} GB/s = {100 * dec_gbs / HBM_PEAK_GBS:.1f}% of peak; "
        f"step {value:.0f} GB/s")

    cpu = None
    if args.cpu_budget > 0:
        dt, runs, blas = cpu_baseline(wl, args.cpu_budget)
        cpu = {"value": round(unique / dt / 1e9, 4), "unit": "GB/s", "cores": blas, "kind": "oracle",
               "sample": f"whole first layer of the workload ({B} sequences), {runs} oracle passes, "
                         f"{dt:.3f} s per pass; numpy fp64 with {blas} BLAS thread(s) on "
                         f"{len(os.sched_getaffinity(0))} available host cores",
               "tokens_per_s": round(B / dt, 2)}
        log(f"cpu oracle: {dt:.3f} s per pass over {B} sequences ({runs} passes)")

    traffic = load_traffic(c.name) if fused and plan is None else None
    # bytes the kernels read from the pools: each prefix item's shared blocks
    # once, every sequence's own positions after its prefix
    read = per_layer_read(wl, plan, c) if shared else logical
    if plan is not None:
        kernel_desc = ("paged_attn_decode_prefix call: partition kernel"
                       + (" with prefix units" if shared else "") + (" (append fused)" if fused else "")
                       + (" over the live partitions (work list)" if work is not None else "") + " + merge kernel")
    elif fused:
        kernel_desc = ("decode_mfma_kernel with the append fused, one launch per layer" if part == 0 else
                       "append_paged_attn_decode call: partition kernel (append fused) + merge kernel")
    else:
        kernel_desc = ("paged_attn_decode call, one kernel" if part == 0 else
                       "paged_attn_decode call: partition kernel + merge kernel")
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
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
        "launch_bytes": launch_bytes,
        "decode_bytes_logical": logical,
        "decode_bytes_read": read,
        "prefix": None if not shared else {"items": plan.num_items, "max_prefix_len": plan.max_prefix_len,
                                           "prefix_tokens": int(plan.prefix_len.sum())},
        "work_list_entries": None if work is None else int(work.shape[0]),
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(round(traffic)),
                     "kernel": kernel_desc},
        "decode_only_call_us": None if decode_only_us is None else round(decode_only_us, 2),
        "decode_only_hbm_frac": None if decode_only_us is None else round(unique / (decode_only_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "launch": launch,
        "append": "fused into the decode kernel" if fused else "separate kv_append kernel",
        "schedule": ("host dispatch order (pkv_decode_schedule)" if order is not None else "sequence order"),
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

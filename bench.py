#!/usr/bin/env python3
"""Benchmark of the sparse MLA forward (top-k = 2048) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

A step is one sparse_mla_fwd call over one synthetic batch (index
compaction + gather + QK^T + softmax + PV + split merge when the plan splits).
Inputs are resident in HBM before timing starts.  K steps are timed with HIP
events on the stream the library launches on, bracketed by device syncs.
Prints ONE JSON line.

Default run: the headline line is the largest single-GPU workload, c5_fp8
(32768 query rows, h=8, fp8 latent cache, top-k 2048): throughput in
query-tokens/s, the attention kernel's roofline (per-launch durations from
HIP events around each launch, HBM-bound), the kernel after evicting the
caches, and the CPU oracle (fp32) timed on a bounded sample of the same
workload on this host.  The same line carries two more measured workloads
under their own keys, each with its own roofline: "c4_long_prefill"
(16384 rows, h=64, bf16: the MFMA-bound target) and "c2_decode" (32 rows,
h=8, split-KV + merge, also replayed from a HIP graph).  For context it also
reports the rates plain torch copy and read kernels reach on this GPU
("measured_bandwidth"); every roofline fraction stays against the published
peak.

Workloads (synthetic, seeded; `--workload` runs one of them alone):
  c5_fp8               32768 rows over 16 sequences (histories 8192..131072), h=8, fp8 cache
                       (c5_fp8_nope: the same with NoPE rows of 512 scaled codes)
  c2_decode            32 rows x 1 query, h=8, 16384-token contexts
  c1_tiny              64 rows, h=8, topk=128
  c3_h{8,16,32,64}     4096 rows over 8 x (8192 + 512) tokens; suffix _pad64 for the padded tiling,
                       _nope for the NoPE geometry (512-wide rows, no rope part)
  c4_long_prefill      16384 rows, h=64, 65536-token history, locality-biased indices
  dense_8x2048         the dense causal entry point on 8 prefill chunks of 2048 tokens
                       from position 0, h=8 (every prefix within top-k)
  topk_4096x65536      the per-row top-k selection: 4096 rows of 65536 fp32 scores
                       (N(0,1) from a seeded device generator), k = 2048
  indexer_4096x65536   the indexer step: MQA logits (64 heads x 128 dims) of 4096 rows against
                       their causal 65536-key history, then top-k 2048
  plan_sweep           native vs padded head tiles and automatic vs no KV splits at T = 16..512,
                       h = 8 / 16 / 32 (the dispatch plan's crossovers)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse MLA fwd: query-tokens/s + gathered-KV GB/s & MFMA % of peak, topk=2048"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="headline",
                    help="headline (c5_fp8 line + c4_long_prefill and c2_decode keys) or one workload")
    ap.add_argument("--splits", type=int, default=0, help="0 = automatic plan")
    ap.add_argument("--variant", type=int, default=0)
    ap.add_argument("--gather-order", default="auto", choices=["auto", "list", "slot"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cold-launches", type=int, default=10)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--copy-reference", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (calibrates HBM byte counters)")
    return ap.parse_args()


def workload(name):
    from sparse_mla_attention_04_amd import inputs as G
    tiling = "native"
    rope = 64
    if name.endswith("_nope"):
        rope = 0
        name = name[:-len("_nope")]
    if name.endswith("_pad64"):
        tiling = "pad64"
        name = name[:-len("_pad64")]
    if name.startswith("c3_h"):
        h = int(name[len("c3_h"):])
        case = G.make_config("c3_sweep", rope_dims=rope).with_heads(h)
        return case, tiling, "c3_sweep" if rope else "c3_sweep_nope"
    if name in ("c1_tiny", "c2_decode", "c4_long_prefill", "c5_fp8") and rope:
        return G.make_config(name), tiling, name
    if name == "c5_fp8" and not rope:
        return G.make_config(name, rope_dims=0), tiling, "c5_fp8_nope"
    if name == "dense_8x2048" and rope:
        return G.build_case(name, seed=1006, hist=[0] * 8, new=[2048] * 8, num_heads=8, topk=2048), tiling, name
    raise SystemExit("unknown workload %s" % name)


def algorithmic_counts(case):
    """Valid (gathered) rows per call, from the index lists as the library sees them."""
    idx = case.topk_idx[:, :case.topk]
    P = case.page_size
    valid = idx >= 0
    j = np.where(valid, idx, 0).astype(np.int64)
    blk = j // P
    valid &= blk < case.block_table.shape[1]
    page = case.block_table[case.token_seq[:, None], np.minimum(blk, case.block_table.shape[1] - 1)]
    valid &= (page >= 0) & (page < case.num_pages)
    return int(valid.sum())


def counted_traffic(workload_name, source="smla_fwd.hip", kernel="smla_fwd<"):
    """HBM bytes per launch of the workload's dominant kernel (name containing
    `kernel`) from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (copy-calibrated), or None when no counters exist for this workload or the
    kernel's source file changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s.json" % workload_name)
    src = os.path.join(ROOT, "sparse_mla_attention_04_amd", "csrc", source)
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        rec = json.load(f)
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec.get("kernel_source_sha256"):
            return None, "stale: kernel source changed since %s" % rec.get("commit")
    for name, v in rec["kernels"].items():
        if kernel in name:
            return v["fetch_bytes"] + v["write_bytes"], "fetch %.0f + write %.0f B (copy-calibrated, %s)" % (
                v["fetch_bytes"], v["write_bytes"], os.path.basename(path))
    return None, None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(case, seconds):
    """The oracle, as it stands, in fp32 on a bounded sample of the
    workload's rows (random order, cycling), on this host's cores."""
    from oracle import sparse_mla_oracle as O
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = 1
    T = case.num_tokens
    rng = np.random.default_rng(0)
    order = rng.permutation(T)
    kw = dict(topk=case.topk, scale=case.scale, kv_format=case.kv_format, page_size=case.page_size,
              index_mode="logical", block_table=case.block_table, token_seq=case.token_seq, dtype=np.float32)
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        rows = [int(order[(done + i) % T]) for i in range(8)]
        O.sparse_mla_forward(case.q, case.kv, case.topk_idx, rows=rows, **kw)
        done += len(rows)
    el = time.perf_counter() - t0
    return {"value": round(done / el, 2), "unit": "query-tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "extrapolated_full_config_s": float("%.3g" % (T * el / done)),
            "sample": "%d query rows of %s (random order over all %d rows) in %.1f s; numpy oracle in fp32 "
                      "(per-row Python gather, BLAS with %d threads)" % (done, case.name, T, el, threads)}


def measured_bandwidth(nbytes=1 << 31, reps=10):
    """Rates of plain torch kernels on this GPU over 2 GiB (more than the L2s
    and the MALL hold): a device copy (bytes read plus bytes written per
    second) and a read-only reduction.  Context beside the published 8 TB/s
    that roofline.frac is taken against; not used in any fraction."""
    import torch
    a = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)

    def rate(fn, moved):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return moved / (float(np.median(ts)) * 1e-3) / 1e9

    copy = rate(lambda: b.copy_(a), 2 * nbytes)
    read = rate(lambda: a.sum(), nbytes)
    del a, b
    torch.cuda.empty_cache()
    return {"copy_GBps": round(copy, 1), "read_GBps": round(read, 1), "bytes": nbytes,
            "kernels": "torch copy_ (read + write counted) and sum (read) over 2 GiB fp32, median of %d" % reps}


def bench_topk(args):
    """The indexer's top-k step alone: rows/s, against HBM (one read of the
    scores plus the index write per launch)."""
    import torch
    from sparse_mla_attention_04_amd import binding as B
    T, N, k = 4096, 65536, 2048
    g = torch.Generator(device="cuda")
    g.manual_seed(1007)
    scores = torch.randn((T, N), generator=g, device="cuda", dtype=torch.float32)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    step = lambda: B.topk(scores, k, out=idx)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    algo = T * N * 4 + T * k * 4
    achieved = algo / (ms * 1e-3) / 1e9
    traffic, traffic_note = counted_traffic("topk_4096x65536", "smla_topk.hip", "smla_topk_kernel")
    res = {"metric": "sparse MLA indexer top-k: query rows/s", "value": round(T / (ms * 1e-3), 1),
           "unit": "query-rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic (seeded device N(0,1))",
           "config": {"workload": "topk_4096x65536", "num_rows": T, "num_keys": N, "k": k},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBPS, 4),
                        "traffic": None if traffic is None else round(traffic), "traffic_note": traffic_note,
                        "kernel": "smla_topk_kernel", "kernel_us": round(ms * 1e3, 2),
                        "algorithmic_bytes": algo}}
    print(json.dumps(res), flush=True)


def run_workload(args, name, *, graph, cold_launches):
    """Time one workload: K steps (value), per-launch kernel durations
    (roofline), optional HIP-graph replay (checked bit for bit) and cold-cache
    launches.  Returns (result dict, case)."""
    import torch
    from sparse_mla_attention_04_amd import binding as B
    from sparse_mla_attention_04_amd.inputs import DeviceCase as Dev

    t_gen = time.perf_counter()
    case, tiling, wl_name = workload(name)
    dev = Dev(case)
    t_gen = time.perf_counter() - t_gen
    T, h = case.num_tokens, case.num_heads
    q = dev.q[:, :h, :]
    out = torch.empty((T, h, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, h), dtype=torch.float32, device="cuda")
    p = B.params_for(q, dev.kv, dev.idx, out, lse, topk=case.topk, scale=case.scale, page_size=case.page_size,
                     kv_format=case.kv_format, block_table=dev.bt, token_seq=dev.ts, tiling=tiling,
                     num_splits=args.splits, kernel_variant=args.variant, gather_order=args.gather_order)
    pl = B.plan(p)
    ws = B.workspace_for(p, "cuda")
    pws = torch.empty(max(16, pl.partials_bytes), dtype=torch.uint8, device="cuda")

    dense = wl_name.startswith("dense")
    if dense:
        counts = np.bincount(case.token_seq, minlength=case.block_table.shape[0])
        d_qs = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
        d_pos = torch.from_numpy(case.positions.astype(np.int32)).cuda()

    def step():
        if dense:
            B.dense_fwd(q, dev.kv, out, lse, block_table=dev.bt, query_start=d_qs, positions=d_pos,
                        scale=case.scale, page_size=case.page_size)
            return
        B.fwd(q, dev.kv, dev.idx, out, lse, topk=case.topk, scale=case.scale, workspace=ws,
              block_table=dev.bt, token_seq=dev.ts, params=p)

    def kernel_only():
        if pl.num_splits > 1 and not dense:
            B.fwd_partials(q, dev.kv, dev.idx, pws, topk=case.topk, scale=case.scale, block_table=dev.bt,
                           token_seq=dev.ts, params=p)
        else:
            step()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # ---- dominant kernel: per-launch durations (events around each launch,
    #      on torch's current stream, which is the stream the library launches on)
    K2 = max(20, min(args.steps, 500))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K2)]
    for a, b in evs:
        a.record()
        kernel_only()
        b.record()
    torch.cuda.synchronize()
    kern_all = np.array([a.elapsed_time(b) for a, b in evs])
    kern_ms = float(np.mean(kern_all))

    # ---- the same step replayed from a HIP graph (launch overhead of the
    #      serving setting); every replay must reproduce the eager result bit for bit
    graph_res = None
    if graph and not args.no_graph:
        step()
        torch.cuda.synchronize()
        ref_out, ref_lse = out.clone(), lse.clone()
        # one graph holds GSTEPS consecutive calls (a serving step captures every
        # layer's call in one graph), so a replay's launch cost is shared
        GSTEPS = 10
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(2):
                step()
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            for _ in range(GSTEPS):
                step()
        checked = 0
        for _ in range(3):
            out.zero_()
            lse.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            if not (torch.equal(out, ref_out) and torch.equal(lse, ref_lse)):
                raise SystemExit("graph replay differs from the eager result")
            checked += 1
        for _ in range(args.warmup):
            g.replay()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        reps = max(1, args.steps // GSTEPS)
        g0.record()
        for _ in range(reps):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / (reps * GSTEPS)
        graph_res = {"ms_per_step": round(gms, 6), "query_tokens_per_s": round(T / (gms * 1e-3), 1),
                     "calls_per_graph": GSTEPS, "replays": reps, "replays_checked_bitwise": checked}
        del g

    # ---- same kernel after evicting caches (1 GiB read between launches, not timed;
    #      reading leaves no dirty lines behind that the kernel would have to write back)
    cold = []
    if cold_launches > 0:
        flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        for _ in range(cold_launches):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            kernel_only()
            b.record()
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b))
        del flush

    # dense: every row attends to its whole prefix (positions + 1 cache rows)
    n_valid = int((case.positions.astype(np.int64) + 1).sum()) if dense else algorithmic_counts(case)
    d_qk = int(case.q.shape[2])
    # fp8 rows: 512 code bytes + 16 bytes of block scales + the bf16 rope part
    row_bytes = 2 * d_qk if case.kv_format == "bf16" else 512 + 16 + 2 * (d_qk - 512)
    gathered = n_valid * row_bytes
    flops = n_valid * h * 2 * (d_qk + 512)
    tokens_per_s = T / (ms_per_step * 1e-3)
    traffic, traffic_note = counted_traffic(name)
    hbm_bound = h < 64 and not dense
    if hbm_bound:
        achieved = gathered / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None}
        if achieved > HBM_PEAK_GBPS:
            # the pool is served from L2 / MALL across query rows: the gathered-byte rate
            # is an effective (cache-served) rate, not an HBM fraction
            roof["effective_cache_served"] = True
            roof["frac"] = None
            roof["frac_counted_hbm"] = (round(traffic / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
                                        if traffic is not None else None)
            roof["mfma_frac_real_heads"] = round(flops / (kern_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
    else:
        achieved = flops / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None}
    roof["traffic"] = None if traffic is None else round(traffic)
    roof["traffic_note"] = traffic_note
    roof["kernel"] = "smla_fwd" + (" (dense causal)" if dense else "" if pl.num_splits == 1 else " (split partials)")
    roof["kernel_us"] = round(kern_ms * 1e3, 2)
    roof["kernel_us_p10_p50_p90"] = [round(float(np.percentile(kern_all, q_)) * 1e3, 2) for q_ in (10, 50, 90)]
    roof["launches_timed"] = K2
    roof["algorithmic_bytes"] = gathered
    roof["algorithmic_flops"] = flops
    roof["per_unit"] = ("one valid gathered row: %d B, %d flop (2 x h x (%d + 512))"
                        % (row_bytes, h * 2 * (d_qk + 512), d_qk))

    config = ({"workload": wl_name, "entry": "sparse_mla_fwd",
               "num_tokens": T, "num_heads": h, "topk": case.topk,
               "kv_format": case.kv_format, "page_size": case.page_size, "tiling": tiling,
               "num_splits": pl.num_splits, "kernel_variant": pl.kernel_variant,
               "gather_order": {1: "list", 2: "slot"}[pl.gather_order],
               "grid": pl.grid, "threads": pl.threads} if not dense else
              {"workload": wl_name, "entry": "sparse_mla_dense_fwd", "num_tokens": T, "num_heads": h,
               "kv_format": case.kv_format, "page_size": case.page_size,
               "rows_per_work_group": 64 // h, "kernel": "pipelined h=64 schedule, (row, head) query slots",
               "grid": ((T + 64 // h - 1) // (64 // h) + case.block_table.shape[0] + 7) // 8 * 8, "threads": 256})
    res = {
        "value": round(tokens_per_s, 1),
        "unit": "query-tokens/s",
        "ms_per_step": round(ms_per_step, 6),
        "steps": args.steps,
        "dtype": "fp8_e4m3+bf16" if case.kv_format == "fp8" else "bf16",
        "config": config,
        "gathered_GBps_per_step": round(gathered / (ms_per_step * 1e-3) / 1e9, 1),
        "mfma_frac_per_step": round(flops / (ms_per_step * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 5),
        "wall_s_timed": round(wall, 4),
        "input_generation_s": round(t_gen, 1),
        "roofline": roof,
        "graph": graph_res,
    }
    if cold:
        cold_ms = float(np.median(cold))
        res["cold_cache"] = {"kernel_us_median": round(cold_ms * 1e3, 2), "launches": len(cold),
                             "gathered_GBps": round(gathered / (cold_ms * 1e-3) / 1e9, 1),
                             "hbm_frac": round(gathered / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                             "note": "1 GiB read between launches to evict L2 and MALL"}
    del out, lse, ws, pws, dev, q
    torch.cuda.empty_cache()
    return res, case


DTYPE_NOTE = {"fp8_e4m3+bf16": "fp8 e4m3 latent cache dequantised exactly to bf16; bf16 MFMA with fp32 "
                               "accumulation and fp32 softmax",
              "bf16": "bf16 cache and MFMA with fp32 accumulation and fp32 softmax"}


def bench_indexer(args):
    """The indexer step: MQA logits (sparse_mla_indexer_logits) then top-k
    (sparse_mla_topk) for 4096 query rows at the last positions of a
    65536-key history, H = 64 heads of 128 dims, k = 2048.  The logits kernel
    is MFMA-bound: algorithmic flops 2 * H * 128 per (row, history key)."""
    import torch
    from sparse_mla_attention_04_amd import binding as B
    from sparse_mla_attention_04_amd import inputs as G
    c = G.make_indexer_case("indexer_4096x65536", seed=1008, num_rows=4096, n_keys=65536, num_heads=64)
    T, N, H = c.num_rows, c.n_keys, c.num_heads
    q = torch.from_numpy(c.q.view(np.int16)).cuda().view(torch.bfloat16)
    k = torch.from_numpy(c.k.view(np.int16)).cuda().view(torch.bfloat16)
    w = torch.from_numpy(c.w).cuda()
    lens = torch.from_numpy(c.lens).cuda()
    logits = torch.empty((T, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, c.topk), dtype=torch.int32, device="cuda")

    def logits_only():
        B.indexer_logits(q, k, w, logits, lens=lens)

    def step():
        logits_only()
        B.topk(logits, c.topk, lens=lens, out=idx)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    K2 = max(20, min(args.steps, 200))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K2)]
    for a_, b_ in evs:
        a_.record()
        logits_only()
        b_.record()
    torch.cuda.synchronize()
    kern = np.array([a_.elapsed_time(b_) for a_, b_ in evs])
    kern_ms = float(np.mean(kern))
    pairs = int(np.clip(c.lens, 0, N).astype(np.int64).sum())
    flops = pairs * H * 128 * 2
    achieved = flops / (kern_ms * 1e-3) / 1e12
    res = {"metric": "sparse MLA indexer (MQA logits + top-k): query rows/s", "value": round(T / (ms * 1e-3), 1),
           "unit": "query-rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic (seeded N(0,1) q, k; N(0,1)/sqrt(H) weights)",
           "config": {"workload": "indexer_4096x65536", "num_rows": T, "n_keys": N, "num_heads": H,
                      "head_dim": 128, "topk": c.topk, "lens": "causal: positions 61440..65535 + 1"},
           "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                        "kernel": "smla_indexer_logits", "kernel_us": round(kern_ms * 1e3, 2),
                        "kernel_us_p10_p50_p90": [round(float(np.percentile(kern, q_)) * 1e3, 2) for q_ in (10, 50, 90)],
                        "algorithmic_flops": flops,
                        "per_unit": "one (row, history key) pair: 2 x H x 128 flop"},
           "topk_us_per_step": round(ms * 1e3 - kern_ms * 1e3, 2)}
    print(json.dumps(res), flush=True)


def bench_plan_sweep(args):
    """The dispatch plan's choices at small batches (native head tiles vs
    padding to 64 heads, automatic KV splits vs none): T decode rows spread
    over the c2_decode pool (32 sequences x 16384 tokens, top-k 2048), h in
    {8, 16, 32}.  Prints one JSON line with the step time of every variant."""
    import torch
    from sparse_mla_attention_04_amd import binding as B
    from sparse_mla_attention_04_amd import inputs as G
    from sparse_mla_attention_04_amd.inputs import DeviceCase as Dev
    rows = []
    for T in (16, 32, 64, 128, 256, 512):
        nseq = min(T, 32)
        per = T // nseq
        case = G.build_case("plan_sweep_T%d" % T, seed=1009, hist=[16384 - per] * nseq, new=[per] * nseq,
                            num_heads=32, topk=2048)
        dev = Dev(case)
        for h in (8, 16, 32):
            q = dev.q[:, :h, :]
            out = torch.empty((T, h, 512), dtype=torch.bfloat16, device="cuda")
            lse = torch.empty((T, h), dtype=torch.float32, device="cuda")
            for tiling, splits in (("native", 0), ("pad64", 0), ("native", 1), ("pad64", 1)):
                p = B.params_for(q, dev.kv, dev.idx, out, lse, topk=case.topk, scale=case.scale,
                                 block_table=dev.bt, token_seq=dev.ts, tiling=tiling, num_splits=splits)
                pl = B.plan(p)
                ws = B.workspace_for(p, "cuda")
                step = lambda: B.fwd(q, dev.kv, dev.idx, out, lse, topk=case.topk, scale=case.scale, workspace=ws,
                                     block_table=dev.bt, token_seq=dev.ts, params=p)
                for _ in range(args.warmup):
                    step()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(args.steps):
                    step()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) / args.steps * 1e3
                rows.append({"T": T, "h": h, "tiling": tiling, "splits_requested": splits or "auto",
                             "num_splits": pl.num_splits, "kernel_variant": pl.kernel_variant, "us_per_step": round(us, 2)})
                print("plan sweep T=%d h=%d %s splits=%s -> S=%d v%d %.2f us" % (
                    T, h, tiling, splits or "auto", pl.num_splits, pl.kernel_variant, us), file=sys.stderr, flush=True)
        del dev
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "sparse MLA fwd: plan sweep, us per step", "unit": "us", "steps": args.steps,
                      "warmup": args.warmup, "config": {"workload": "plan_sweep", "pool": "32 x 16384 tokens",
                                                         "topk": 2048}, "rows": rows}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs the sparse MLA forward on a single "
              "MI355X (no collectives); --gpus %d is not supported." % args.gpus, flush=True)
        sys.exit(2)
    import torch
    if args.copy_reference:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_reference_bytes_read": src.numel() * 4, "launches": 5}), flush=True)
        return
    if args.workload == "topk_4096x65536":
        return bench_topk(args)
    if args.workload == "indexer_4096x65536":
        return bench_indexer(args)
    if args.workload == "plan_sweep":
        return bench_plan_sweep(args)

    headline = args.workload == "headline"
    main_name = "c5_fp8" if headline else args.workload
    print("bench: %s" % main_name, file=sys.stderr, flush=True)
    res_main, case_main = run_workload(args, main_name, graph=not headline and main_name == "c2_decode",
                                       cold_launches=args.cold_launches)
    extras = {}
    if headline:
        for name, graph in (("c4_long_prefill", False), ("c2_decode", True)):
            print("bench: %s" % name, file=sys.stderr, flush=True)
            r, _ = run_workload(args, name, graph=graph, cold_launches=args.cold_launches)
            r.pop("steps", None)
            extras[name] = r
    res = {
        "metric": METRIC,
        "value": res_main["value"],
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res_main["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res_main["dtype"],
        "dtype_note": DTYPE_NOTE[res_main["dtype"]],
        "data": "synthetic (seeded; shapes and distributions of the workload, no dataset)",
        "config": res_main["config"],
    }
    for k in ("gathered_GBps_per_step", "mfma_frac_per_step", "wall_s_timed", "input_generation_s", "roofline",
              "graph", "cold_cache"):
        if k in res_main:
            res[k] = res_main[k]
    res.update(extras)
    print("bench: measured bandwidth", file=sys.stderr, flush=True)
    res["measured_bandwidth"] = measured_bandwidth()
    if not args.no_cpu_baseline:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(case_main, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

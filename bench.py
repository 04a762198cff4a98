#!/usr/bin/env python3
"""Benchmark of the sparse MLA forward (top-k = 2048) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload c2_decode]

A step is one sparse_mla_fwd call over one synthetic batch (index
compaction + gather + QK^T + softmax + PV + split merge when the plan splits).
Inputs are resident in HBM before timing starts.  K steps are timed with HIP
events on the stream the library launches on, bracketed by device syncs.
Prints ONE JSON line: throughput in query-tokens/s, the dominant kernel's
roofline (per-launch durations from events around each launch), the same
step replayed from a HIP graph (checked bit for bit against the eager
result), the kernel after evicting the caches (1 GiB read between launches),
and the CPU oracle timed on a bounded sample of the same workload on this
host.

Workloads (synthetic, seeded; `--workload`):
  c2_decode (default)  32 rows x 1 query, h=8, 16384-token contexts
  c1_tiny              64 rows, h=8, topk=128
  c3_h{8,16,32,64}     4096 rows over 8 x (8192 + 512) tokens; suffix _pad64 for the padded tiling,
                       _nope for the NoPE geometry (512-wide rows, no rope part)
  c4_long_prefill      16384 rows, h=64, 65536-token history, locality-biased indices
  dense_8x2048         the dense causal entry point on 8 prefill chunks of 2048 tokens
                       from position 0, h=8 (every prefix within top-k)
  topk_4096x65536      the per-row top-k selection: 4096 rows of 65536 fp32 scores
                       (N(0,1) from a seeded device generator), k = 2048
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
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="c2_decode")
    ap.add_argument("--splits", type=int, default=0, help="0 = automatic plan")
    ap.add_argument("--variant", type=int, default=0)
    ap.add_argument("--gather-order", default="auto", choices=["auto", "list", "slot"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cold-launches", type=int, default=50)
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


def counted_traffic(workload_name):
    """HBM bytes per launch of the attention kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs (copy-calibrated), or None when no
    counters exist for this workload or the kernel source changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s.json" % workload_name)
    src = os.path.join(ROOT, "sparse_mla_attention_04_amd", "csrc", "smla_fwd.hip")
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        rec = json.load(f)
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec.get("kernel_source_sha256"):
            return None, "stale: kernel source changed since %s" % rec.get("commit")
    for name, v in rec["kernels"].items():
        if "smla_fwd<" in name:
            return v["fetch_bytes"] + v["write_bytes"], "fetch %.0f + write %.0f B (copy-calibrated, %s)" % (
                v["fetch_bytes"], v["write_bytes"], os.path.basename(path))
    return None, None


def cpu_baseline(case, seconds):
    """The oracle, as it stands, on a bounded sample of the workload's rows."""
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
              index_mode="logical", block_table=case.block_table, token_seq=case.token_seq)
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        rows = [int(order[(done + i) % T]) for i in range(8)]
        O.sparse_mla_forward(case.q, case.kv, case.topk_idx, rows=rows, **kw)
        done += len(rows)
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "query-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d query rows (random order, cycling over all %d rows of the workload) in %.1f s, "
                      "numpy fp64 oracle" % (done, T, el)}


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
    res = {"metric": "sparse MLA indexer top-k: query rows/s", "value": round(T / (ms * 1e-3), 1),
           "unit": "query-rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic (seeded device N(0,1))",
           "config": {"workload": "topk_4096x65536", "num_rows": T, "num_keys": N, "k": k},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                        "kernel": "smla_topk_kernel", "kernel_us": round(ms * 1e3, 2),
                        "algorithmic_bytes": algo}}
    print(json.dumps(res), flush=True)


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
    from sparse_mla_attention_04_amd import binding as B
    from sparse_mla_attention_04_amd.inputs import DeviceCase as Dev

    if args.workload == "topk_4096x65536":
        return bench_topk(args)
    case, tiling, wl_name = workload(args.workload)
    dev = Dev(case)
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

    # ---- dominant kernel: per-launch durations (events around each launch)
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
    graph = None
    if not args.no_graph:
        step()
        torch.cuda.synchronize()
        ref_out, ref_lse = out.clone(), lse.clone()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(2):
                step()
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
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
        g0.record()
        for _ in range(args.steps):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / args.steps
        graph = {"ms_per_step": round(gms, 6), "query_tokens_per_s": round(T / (gms * 1e-3), 1),
                 "replays_checked_bitwise": checked}
        del g

    # ---- same kernel after evicting caches (1 GiB read between launches, not timed;
    #      reading leaves no dirty lines behind that the kernel would have to write back)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    cold = []
    for _ in range(args.cold_launches):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        kernel_only()
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    cold_ms = float(np.median(cold))
    del flush

    # dense: every row attends to its whole prefix (positions + 1 cache rows)
    n_valid = int((case.positions.astype(np.int64) + 1).sum()) if dense else algorithmic_counts(case)
    d_qk = int(case.q.shape[2])
    row_bytes = 2 * d_qk if case.kv_format == "bf16" else 656
    gathered = n_valid * row_bytes
    flops = n_valid * h * 2 * (d_qk + 512)
    tokens_per_s = T / (ms_per_step * 1e-3)
    hbm_bound = h < 64 and not dense
    if hbm_bound:
        achieved = gathered / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None}
    else:
        achieved = flops / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None}
    traffic, traffic_note = counted_traffic(args.workload)
    roof["traffic"] = None if traffic is None else round(traffic)
    roof["traffic_note"] = traffic_note
    roof["kernel"] = "smla_fwd" + (" (dense causal)" if dense else "" if pl.num_splits == 1 else " (split partials)")
    roof["kernel_us"] = round(kern_ms * 1e3, 2)
    roof["kernel_us_p10_p50_p90"] = [round(float(np.percentile(kern_all, q)) * 1e3, 2) for q in (10, 50, 90)]
    roof["algorithmic_bytes"] = gathered
    roof["algorithmic_flops"] = flops

    res = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl_name, "entry": "sparse_mla_dense_fwd" if dense else "sparse_mla_fwd",
                   "num_tokens": T, "num_heads": h, "topk": case.topk,
                   "kv_format": case.kv_format, "page_size": case.page_size, "tiling": tiling,
                   "num_splits": pl.num_splits, "kernel_variant": pl.kernel_variant,
                   "gather_order": {1: "list", 2: "slot"}[pl.gather_order],
                   "grid": pl.grid, "threads": pl.threads} if not dense else
                  {"workload": wl_name, "entry": "sparse_mla_dense_fwd", "num_tokens": T, "num_heads": h,
                   "kv_format": case.kv_format, "page_size": case.page_size,
                   "rows_per_work_group": 64 // h, "kernel": "pipelined h=64 schedule, (row, head) query slots",
                   "grid": ((T + 64 // h - 1) // (64 // h) + case.block_table.shape[0] + 7) // 8 * 8, "threads": 256},
        "gathered_GBps_per_step": round(gathered / (ms_per_step * 1e-3) / 1e9, 1),
        "mfma_frac_per_step": round(flops / (ms_per_step * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 5),
        "wall_s_timed": round(wall, 4),
        "roofline": roof,
        "graph": graph,
        "cold_cache": {"kernel_us_median": round(cold_ms * 1e3, 2),
                       "gathered_GBps": round(gathered / (cold_ms * 1e-3) / 1e9, 1),
                       "hbm_frac": round(gathered / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                       "note": "1 GiB read between launches to evict L2 and MALL"},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

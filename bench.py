"""Decode-step benchmark of the Locks path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--rank R]

One step = locks_decode_step over the whole batch, with synthetic inputs
already resident in HBM: the page scorer (summary scan), the share-average
combine and top-k selection, and the split-K sparse decode, three launches
on one stream. Every kernel is also timed on its own. The summary build of
the pages that complete in a step is timed in the same run and reported
beside it (it runs when a page completes, off the decode critical path),
together with the one-off build of every page after prefill.

Prints one JSON line. `hbm_roofline_frac_step` is the whole step's
algorithmic bytes (summary records + selected K/V) over its time and the HBM
peak; `roofline` describes the dominant kernel, the page scorer (summary
bytes per launch), and `sparse_decode_roofline` the decode (selected K/V
bytes); `cpu_baseline` times the fp64 CPU oracle on a bounded sample of the
same step.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

METRIC = "decode-step score+select+sparse-attn µs and % HBM roofline, 128K ctx, batch 8"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
N_QUERY_SETS = 8  # query sets rotated through timed steps (default of --query-sets)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=192, help="timed steps, in three windows")
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="llama8b_128k_b8")
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--summary-dtype", choices=("bf16", "f32", "i4"), default=None,
                    help="summary records (default: the workload's); i4 = 4-bit basis, 8-bit "
                         "centroid and coefficients, bf16 scales, reported as workload <name>_i4")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--kv-host", action="store_true",
                    help="hold the K/V pools in pinned host memory: the decode reads the selected pages "
                         "over the host link (the summaries stay in HBM)")
    ap.add_argument("--query-sets", type=int, default=N_QUERY_SETS,
                    help="query sets rotated through the timed steps (1: every step repeats one query)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=24.0,
                    help="CPU time of the oracle baseline (two legs of three runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run 3 plain device copies of MIB MiB "
                         "(reference dispatches for scaling memory counters)")
    ap.add_argument("--full-step", action="store_true",
                    help="instead of the 128K batch-8 layer step: the 32-layer decode step of a 16 x 64K batch "
                         "with the builds of completing pages interleaved (its own JSON line)")
    ap.add_argument("--hot-cache", type=float, default=None, metavar="MULT",
                    help="instead of the layer step: the step with the K/V pools in pinned host memory read "
                         "through the GPU hot-page cache of MULT steps' tiles (its own JSON line)")
    ap.add_argument("--query-rho", type=float, default=0.9,
                    help="--hot-cache: correlation of consecutive steps' queries (AR(1) sequence)")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("STATS_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: turn the rocprofv3 outputs of the commands in profiles/*.md into "
                         "profiles/traffic_<workload>.json and the two summaries")
    return ap.parse_args()


def resolve_workload(args):
    """The named workload with the --rank / --summary-dtype overrides; i4
    summaries are reported under <name>_i4."""
    from sparse_kv_page_amd import synth
    wl = synth.WORKLOADS[args.workload]
    if args.rank is not None:
        wl = wl.with_(rank=args.rank)
    if args.summary_dtype is not None and args.summary_dtype != wl.summary_dtype:
        wl = wl.with_(summary_dtype=args.summary_dtype, name=f"{wl.name}_{args.summary_dtype}")
    return wl


def bench_flags(args):
    """The command-line flags that select the workload (for the recorded commands)."""
    f = []
    if args.workload != "llama8b_128k_b8":
        f.append(f"--workload {args.workload}")
    if args.rank is not None:
        f.append(f"--rank {args.rank}")
    if args.summary_dtype is not None:
        f.append(f"--summary-dtype {args.summary_dtype}")
    return (" " + " ".join(f)) if f else ""


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(resolve_workload(args), bench_flags(args), *args.summarize_profiles)
        return
    if args.full_step or args.hot_cache is not None:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            sys.exit(2)
        full_step(args) if args.full_step else hot_cache_step(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by (sequence, KV head) with no exchange, so N GPUs would run N "
              "independent copies).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_kv_page_amd import locks as L
    from sparse_kv_page_amd import synth

    torch.cuda.set_device(0)
    dev = "cuda"
    wl = resolve_workload(args)
    cfg = L.config_for(wl)
    B, Hkv, Hq, d, P, r, k = (wl.batch, wl.num_kv_heads, wl.num_q_heads, wl.head_dim,
                              wl.page_size, wl.rank, wl.budget_pages)
    print(f"[bench] generating {wl.name} (batch {B}, ctx {wl.seq_lens[0]}, r {r}) on the GPU",
          file=sys.stderr, flush=True)
    data = synth.generate(wl, args.seed, dev)
    q, kp, vp, bt, sl = (data[x] for x in ("q", "k_pool", "v_pool", "block_table", "seq_lens"))
    maxp = wl.max_pages
    pool = L.summary_pool_for(cfg, wl.num_blocks, dev)
    rec_bytes = L.locks_summary_record_bytes(cfg)

    # ---- prefill build of every complete page (one-off) ----
    full_ids = []
    for b in range(B):
        Jc = int(wl.seq_lens[b]) // P
        full_ids.append(bt[b, :Jc])
    full_ids = torch.cat(full_ids).contiguous()
    n_full = full_ids.numel()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    L.locks_build_summaries(cfg, kp, wl.num_blocks, full_ids, n_full, pool)  # warm
    torch.cuda.synchronize()
    e0.record()
    L.locks_build_summaries(cfg, kp, wl.num_blocks, full_ids, n_full, pool)
    e1.record()
    torch.cuda.synchronize()
    prefill_build_ms = e0.elapsed_time(e1)
    print(f"[bench] prefill build of {n_full * Hkv} page tiles: {prefill_build_ms:.2f} ms",
          file=sys.stderr, flush=True)

    # K/V in pinned host memory: the decode reads the selected pages in place
    kp_dec, vp_dec, kv_host = kp, vp, None
    if args.kv_host:
        kh, kp_dec = host_pool(kp)
        vh, vp_dec = host_pool(vp)
        kv_host = (kh, vh)
        print(f"[bench] K/V pools in pinned host memory ({2 * kh.numel() * kh.element_size() / 2**30:.1f} GiB)",
              file=sys.stderr, flush=True)

    # pages completing in a decode step: the current page of every sequence whose
    # length is a multiple of the page size
    step_ids = torch.stack([bt[b, int(wl.seq_lens[b]) // P - 1] for b in range(B)
                            if int(wl.seq_lens[b]) % P == 0]).to(torch.int32).contiguous()
    n_step = step_ids.numel()

    sel = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, d), dtype=synth.torch_dtype(wl.kv_dtype), device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws_bytes = L.locks_workspace_size(cfg, B, maxp)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    scores = torch.empty((B, Hq, maxp), dtype=torch.float32, device=dev)
    sigma = torch.empty((B, Hkv, maxp), dtype=torch.float32, device=dev)

    # Query sets rotated through the timed steps (each step is a new decode
    # step of the same batch): their selections differ, so the selected K/V
    # of consecutive steps (64 MiB each at the headline) never add up to
    # fewer bytes than the 256 MB last-level cache holds, and no step is
    # served from what an earlier step left there.
    gq = torch.Generator(device=dev)
    gq.manual_seed(args.seed + 1)
    nq = max(1, args.query_sets)
    qsets = [q] + [torch.randn(q.shape, generator=gq, device=dev, dtype=torch.float32).to(q.dtype)
                   for _ in range(nq - 1)]
    sels = [torch.empty_like(sel) for _ in qsets]
    for qi, si in zip(qsets, sels):
        L.locks_score_select(cfg, qi, pool, wl.num_blocks, bt, sl, B, maxp, si, ws, ws_bytes)
    torch.cuda.synchronize()
    distinct_kv = selected_kv_footprint(wl, sels, bt)

    def score(t):
        L.locks_page_score(cfg, qsets[t % nq], pool, wl.num_blocks, bt, sl, B, maxp, scores)

    def select(t):
        L.locks_select_pages(cfg, scores, sl, B, maxp, sel, sigma)

    def decode(t):
        i = t % nq
        L.locks_sparse_decode(cfg, qsets[i], kp_dec, vp_dec, wl.num_blocks, bt, sl, sels[i], B, maxp, out, lse,
                              ws, ws_bytes)

    def staged(t):
        # page scoring -> combine + selection -> sparse decode, three launches
        L.locks_page_score(cfg, qsets[t % nq], pool, wl.num_blocks, bt, sl, B, maxp, scores)
        L.locks_select_pages(cfg, scores, sl, B, maxp, sel, sigma)
        L.locks_sparse_decode(cfg, qsets[t % nq], kp_dec, vp_dec, wl.num_blocks, bt, sl, sel, B, maxp,
                              out, lse, ws, ws_bytes)

    def step(t):
        # the whole step through the library's one-call entry point
        L.locks_decode_step(cfg, qsets[t % nq], pool, kp_dec, vp_dec, wl.num_blocks, bt, sl, B, maxp,
                            sel, out, lse, ws, ws_bytes)

    # throttle counters: a sampled read over the whole measured part (taken
    # before the warm-up and after the last timed window, so its ~100 ms of
    # host time never precede a timed window) and a quick one per window
    throttle = ThrottleMonitor()
    region0 = throttle.read_sampled()
    for t in range(args.warmup):
        step(t)
        staged(t)
    torch.cuda.synchronize()

    def windows(fn, n_steps, n_windows=3):
        """n_steps launches of fn in n_windows timed windows (HIP events on
        torch's stream, which is the stream every call above enqueues on),
        synchronised between windows. Returns the per-window ms per step and
        each window's throttle record."""
        sizes = [n_steps // n_windows + (1 if i < n_steps % n_windows else 0) for i in range(n_windows)]
        per, thr = [], []
        t = 0
        for n in sizes:
            if n == 0:
                continue
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            before = throttle.read()
            e0.record()
            for _ in range(n):
                fn(t)
                t += 1
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / n)
            thr.append(throttle.delta(before, throttle.read()))
        return per, thr, sizes

    # ---- timed region: exactly K steps, in three windows ----
    wall0 = time.perf_counter()
    step_win, step_thr, win_sizes = windows(step, args.steps)
    wall1 = time.perf_counter()
    step_ms = sum(w * n for w, n in zip(step_win, win_sizes)) / args.steps

    # ---- the same step as three launches, and each launch on its own: K
    # back-to-back launches on the same stream, HIP events around ----
    staged_win, _, _ = windows(staged, args.steps)
    staged_ms = sum(w * n for w, n in zip(staged_win, win_sizes)) / args.steps
    stage_us = {"decode_step": 1e3 * step_ms}
    score(0)
    for name, fn in (("page_score", score), ("select", select), ("sparse_decode", decode)):
        w, _, _ = windows(fn, args.steps)
        stage_us[name] = 1e3 * sum(x * n for x, n in zip(w, win_sizes)) / args.steps

    # ---- summary build of the pages that complete in a step (off the decode path) ----
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    build_ms = 0.0
    if n_step:
        for _ in range(3):
            L.locks_build_summaries(cfg, kp, wl.num_blocks, step_ids, n_step, pool)
        b0.record()
        for _ in range(args.steps):
            L.locks_build_summaries(cfg, kp, wl.num_blocks, step_ids, n_step, pool)
        b1.record()
        torch.cuda.synchronize()
        build_ms = b0.elapsed_time(b1) / args.steps
    stage_us["build_step"] = 1e3 * build_ms
    throttle_region = throttle.delta(region0, throttle.read_sampled())

    summary_bytes, kv_bytes = algorithmic_bytes(wl, rec_bytes)
    step_bytes = summary_bytes + kv_bytes
    step_gbs = step_bytes / (step_ms * 1e-3) / 1e9
    # the dual Gram M = D D^T of each (page, KV head) tile on the matrix cores:
    # three bf16 products (hi.hi, hi.lo, lo.hi of the centred keys) of 2 P^2 d
    # flops each for bf16 keys, one fp32 product for fp32 keys
    gram_flops = (3.0 if wl.kv_dtype == "bf16" else 1.0) * 2.0 * P * P * d * n_full * Hkv
    build_tflops = gram_flops / (prefill_build_ms * 1e-3) / 1e12
    copy = copy_bandwidth(dev)

    if args.copy_calibration > 0:
        nb = args.copy_calibration << 20
        src = torch.ones(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- CPU oracle on a bounded sample of the same step ----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, cfg, data, args.cpu_seconds, step_bytes)

    us = [round(1e3 * w, 3) for w in step_win]
    ok = [w for w, t in zip(us, step_thr) if not (t or {}).get("throttled")]
    res = {
        "metric": METRIC,
        "value": round(step_ms * 1e3, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.kv_dtype,
        "data": "synthetic",
        "config": {"workload": wl.name + ("_kvhost" if kv_host is not None else ""), "batch": B,
                   "context_tokens": int(wl.seq_lens[0]),
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "page_size": P, "rank": r,
                   "budget_tokens": k * P, "summary_dtype": wl.summary_dtype,
                   "query_sets": nq, "parallelism": "single-gpu"},
        "hbm_roofline_frac_step": round(step_gbs / HBM_PEAK_GBS, 4),
        "step_algorithmic_bytes": step_bytes,
        "step_achieved_GBps": round(step_gbs, 1),
        "windows": {"steps_per_window": win_sizes, "us_per_step": us,
                    "median_us": round(statistics.median(us), 3), "mean_us": round(statistics.mean(us), 3),
                    "sd_us": round(statistics.stdev(us), 3) if len(us) > 1 else 0.0,
                    "throttle": step_thr, "unthrottled_mean_us": round(statistics.mean(ok), 3) if ok else None,
                    "throttle_whole_run": throttle_region},
        "measured_copy_GBps": copy,
        "roofline": roofline("page_score", wl, summary_bytes, stage_us["page_score"]),
        "sparse_decode_roofline": (roofline("sparse_decode", wl, kv_bytes, stage_us["sparse_decode"])
                                   if kv_host is None else
                                   {"bound": "host link", "kernel": "sparse_decode",
                                    "achieved": round(kv_bytes / (stage_us["sparse_decode"] * 1e-6) / 1e9, 1),
                                    "unit": "GB/s", "algorithmic_bytes_per_launch": kv_bytes,
                                    "avg_launch_us": round(stage_us["sparse_decode"], 3)}),
        "selected_kv_bytes_across_query_sets": distinct_kv,
        "kv_resident": "host" if kv_host is not None else "hbm",
        "staged_step_us": round(staged_ms * 1e3, 3),
        "stages_us": {n: round(v, 3) for n, v in stage_us.items()},
        "step_with_build_us": round(step_ms * 1e3 + stage_us["build_step"], 3),
        "build": {"pages_per_step": int(n_step) * Hkv, "step_build_us": round(stage_us["build_step"], 3),
                  "prefill_page_tiles": int(n_full) * Hkv, "prefill_ms": round(prefill_build_ms, 3),
                  "gram_TFLOPs": round(build_tflops, 3),
                  "gram_mfma_frac": round(build_tflops / BF16_MFMA_PEAK_TFLOPS, 5)},
        "wall_s_timed": round(wall1 - wall0, 4),
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def full_step(args):
    """The decode step of a whole model (sparse_kv_page_amd.synth.FULL_STEP:
    32 attention layers of a batch of 16 sequences of ~64K tokens, sequence s
    4 s tokens longer, so one sequence completes a page every 4 steps; r = 4,
    k = 32). Keys and values of every layer come from the low-rank generator;
    all layers' K/V live in one paged pool (~138 GB) and their summaries in one
    summary pool. A step = locks_decode_step for every layer, the build of the
    page the step's token completes in every layer (block ids gathered from a
    step table by a step counter kept on the device, so the step's launches
    are the same every step), and the length increment, on one stream. Timed
    eagerly, then replayed from one captured HIP graph that holds the whole
    step, builds included."""
    import torch

    from sparse_kv_page_amd import locks as L
    from sparse_kv_page_amd import synth

    sh = synth.FULL_STEP
    nl, B, Hkv, G, d, P, r, k = (sh["layers"], sh["batch"], sh["kv_heads"], sh["group"], sh["head_dim"],
                                 sh["page_size"], sh["rank"], sh["budget_pages"])
    Hq = Hkv * G
    steps, warm = args.steps, args.warmup
    total = 2 * warm + 2 * steps + 2  # eager warm-up and timed steps, capture warm-up, graph warm-up and timed
    torch.cuda.set_device(0)
    dev = "cuda"
    t0 = time.perf_counter()
    inp = synth.full_step_inputs(total, seed=args.seed, device=dev,
                                 log=lambda m: print(f"[full] {m} ({time.perf_counter() - t0:.0f} s)",
                                                     file=sys.stderr, flush=True))
    NB, maxp, lens0 = inp["num_blocks"], inp["max_pages"], inp["lens0"]
    cfg = L.make_config(d, P, r, Hq, Hkv, k, "bf16", "bf16", 1.0 / math.sqrt(d))
    kp, vp, bt, q = inp["k_pool"], inp["v_pool"], inp["block_table"], inp["q"]
    spool = L.summary_pool_for(cfg, NB, dev)
    full_ids = torch.cat([bt[layer, s, :lens0[s] // P] for layer in range(nl) for s in range(B)]).contiguous()
    L.locks_build_summaries(cfg, kp, NB, full_ids, full_ids.numel(), spool)
    torch.cuda.synchronize()
    print(f"[full] prefill build of {full_ids.numel() * Hkv} tiles done ({time.perf_counter() - t0:.0f} s)",
          file=sys.stderr, flush=True)
    ws_bytes = L.locks_workspace_size(cfg, B, maxp)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    sel = torch.empty((nl, B, Hkv, k), dtype=torch.int32, device=dev)
    out = torch.empty((nl, B, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((nl, B, Hq), dtype=torch.float32, device=dev)
    seq = torch.tensor(lens0, dtype=torch.int32, device=dev)
    step_idx = torch.zeros(1, dtype=torch.int64, device=dev)
    ids_buf = torch.full((1, nl), -1, dtype=torch.int32, device=dev)
    done = [0]  # steps taken (host count, so the step table is never read past its end)

    def step():
        for layer in range(nl):
            L.locks_decode_step(cfg, q[layer], spool, kp, vp, NB, bt[layer], seq, B, maxp, sel[layer], out[layer],
                                lse[layer], ws, ws_bytes)
        torch.index_select(inp["build_ids"], 0, step_idx, out=ids_buf)
        L.locks_build_summaries(cfg, kp, NB, ids_buf, ids_buf.numel(), spool)
        seq.add_(1)
        step_idx.add_(1)

    def run(n, graph=None):
        assert done[0] + n <= total, "step table exhausted"
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            step() if graph is None else graph.replay()
        e1.record()
        torch.cuda.synchronize()
        done[0] += n
        return e0.elapsed_time(e1) * 1e3 / n

    run(warm)                                      # warm-up (eager)
    eager_us = run(steps)
    # graph of the whole step, builds included
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    done[0] += 1
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    run(warm, graph)                               # warm-up (graph)
    graph_us = run(steps, graph)
    # the build share: the same steps' builds alone
    ids_c = inp["build_ids"].cpu()
    n_build = sum(1 for t in range(warm, warm + steps) if int(ids_c[t, 0]) >= 0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for t in range(warm, warm + steps):
        L.locks_build_summaries(cfg, kp, NB, inp["build_ids"][t], nl, spool)
    e1.record()
    torch.cuda.synchronize()
    build_us = e0.elapsed_time(e1) * 1e3 / steps
    wl = synth.Workload("full_step", B, Hkv, G, d, P, tuple(lens0), r, k, "bf16", "bf16")
    sb, kb = algorithmic_bytes(wl, L.locks_summary_record_bytes(cfg))
    step_bytes = nl * (sb + kb)
    res = {"metric": "full decode step µs (32 layers, builds of completing pages interleaved)",
           "value": round(eager_us, 1), "unit": "us", "n_gpus": 1, "steps": steps, "warmup": warm,
           "higher_is_better": False, "dtype": "bf16", "data": "synthetic (low-rank key generator)",
           "config": {"workload": "full_step", "layers": nl, "batch": B, "context_tokens": lens0[0],
                      "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "page_size": P, "rank": r,
                      "budget_tokens": k * P, "kv_bytes_resident": 2 * kp.numel() * 2},
           "step_algorithmic_bytes": step_bytes,
           "hbm_roofline_frac_step": round(step_bytes / (eager_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "graph_us_per_step": round(graph_us, 1),
           "graph_holds": "every layer's decode step, the step's builds and the length increment",
           "build_us_per_step": round(build_us, 1), "build_share": round(build_us / eager_us, 4),
           "steps_with_a_completing_page": n_build}
    print(json.dumps(res), flush=True)


def hot_cache_step(args):
    """The decode step with the K/V pools in pinned host memory, read through
    the GPU hot-page cache (locks_decode_step_cached, a clock cache of
    (block, KV head) tiles; [Locks] §5.3 Table 3 and App. B.4.2 keep the full
    K/V in host memory and the pages used often in a smaller GPU cache). The
    queries of consecutive steps form an AR(1) sequence (--query-rho), the
    cache holds --hot-cache times one step's tiles. Timed beside the same
    steps without the cache (every selected tile over the host link) and with
    device-resident pools; the hit share is counted over the timed steps, and
    for a few other query correlations over shorter runs."""
    import torch

    from sparse_kv_page_amd import locks as L
    from sparse_kv_page_amd import synth

    torch.cuda.set_device(0)
    dev = "cuda"
    wl = resolve_workload(args)
    cfg = L.config_for(wl)
    B, Hkv, Hq, d, P, k = wl.batch, wl.num_kv_heads, wl.num_q_heads, wl.head_dim, wl.page_size, wl.budget_pages
    data = synth.generate(wl, args.seed, dev)
    q, kp, vp, bt, sl = (data[x] for x in ("q", "k_pool", "v_pool", "block_table", "seq_lens"))
    maxp, NB = wl.max_pages, wl.num_blocks
    pool = L.summary_pool_for(cfg, NB, dev)
    ids = torch.cat([bt[b, :int(wl.seq_lens[b]) // P] for b in range(B)]).contiguous()
    L.locks_build_summaries(cfg, kp, NB, ids, ids.numel(), pool)
    kh, kdev = host_pool(kp)
    vh, vdev = host_pool(vp)
    n = B * Hkv * k
    capacity = int(round(args.hot_cache * n))
    cache = L.HotCache(cfg, NB, capacity, dev)
    tile_bytes = P * d * (2 if wl.kv_dtype == "bf16" else 4)
    print(f"[hot-cache] {wl.name}: K/V in host memory ({2 * kh.numel() * kh.element_size() / 2**30:.1f} GiB), "
          f"cache of {capacity} tiles ({2 * capacity * tile_bytes / 2**30:.2f} GiB)", file=sys.stderr, flush=True)
    sel = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, d), dtype=synth.torch_dtype(wl.kv_dtype), device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws_bytes = L.locks_workspace_size(cfg, B, maxp)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    warm, steps = args.warmup, args.steps
    qs = synth.query_sequence(q, warm + steps, args.query_rho, args.seed)

    def cached(t, qseq=qs):
        L.locks_decode_step_cached(cfg, qseq[t], pool, kdev, vdev, NB, bt, sl, B, maxp, sel, out, lse, cache.buf,
                                   capacity, ws, ws_bytes)

    def uncached(t):
        L.locks_decode_step(cfg, qs[t], pool, kdev, vdev, NB, bt, sl, B, maxp, sel, out, lse, ws, ws_bytes)

    def device(t):
        L.locks_decode_step(cfg, qs[t], pool, kp, vp, NB, bt, sl, B, maxp, sel, out, lse, ws, ws_bytes)

    def timed(fn):
        for t in range(warm):
            fn(t)
        torch.cuda.synchronize()
        per = []
        for w in range(3):  # three windows over consecutive steps
            lo, hi = warm + w * steps // 3, warm + (w + 1) * steps // 3
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for t in range(lo, hi):
                fn(t)
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / (hi - lo))
        return per

    cache.reset()
    for t in range(warm):
        cached(t)
    torch.cuda.synchronize()
    s0 = cache.stats()
    cache_win = []
    for w in range(3):
        lo, hi = warm + w * steps // 3, warm + (w + 1) * steps // 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(lo, hi):
            cached(t)
        e1.record()
        torch.cuda.synchronize()
        cache_win.append(e0.elapsed_time(e1) * 1e3 / (hi - lo))
    s1 = cache.stats()
    st = {key: s1[key] - s0[key] for key in s1}
    served = st["hits"] + st["misses"] + st["refreshes"] + st["shared"]
    hit_share = st["hits"] / served if served else None
    copied = (st["misses"] + st["refreshes"]) / max(1, st["steps"])
    host_win = timed(uncached)
    dev_win = timed(device)
    print(f"[hot-cache] cached {statistics.median(cache_win):.1f} us, uncached host "
          f"{statistics.median(host_win):.1f} us, device {statistics.median(dev_win):.1f} us, hit share "
          f"{hit_share:.3f}", file=sys.stderr, flush=True)

    # hit share for other query correlations (shorter runs, untimed)
    by_rho = {}
    for rho in (0.0, 0.5, 0.9, 0.97):
        qr = synth.query_sequence(q, 96, rho, args.seed + 5)
        cache.reset()
        for t in range(32):
            cached(t, qr)
        torch.cuda.synchronize()
        a = cache.stats()
        for t in range(32, 96):
            cached(t, qr)
        torch.cuda.synchronize()
        b_ = cache.stats()
        srv = sum(b_[x] - a[x] for x in ("hits", "misses", "refreshes", "shared"))
        by_rho[str(rho)] = round((b_["hits"] - a["hits"]) / srv, 4)
    del kh, vh
    med = statistics.median(cache_win)
    res = {"metric": "decode step us, K/V in host memory through the GPU hot-page cache",
           "value": round(statistics.mean(cache_win), 3), "unit": "us", "n_gpus": 1, "steps": steps,
           "warmup": warm, "higher_is_better": False, "dtype": wl.kv_dtype,
           "data": "synthetic (AR(1) queries across steps)",
           "config": {"workload": wl.name + "_hotcache", "batch": B, "context_tokens": int(wl.seq_lens[0]),
                      "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "page_size": P, "rank": wl.rank,
                      "budget_tokens": k * P, "capacity_tiles": capacity,
                      "capacity_steps": args.hot_cache, "cache_GiB": round(2 * capacity * tile_bytes / 2**30, 3),
                      "query_rho": args.query_rho},
           "windows_us": [round(x, 3) for x in cache_win], "median_us": round(med, 3),
           "hit_share": round(hit_share, 4) if hit_share is not None else None,
           "counts_over_timed_steps": st,
           "tiles_copied_per_step": round(copied, 2),
           "host_link_bytes_per_step": int(copied * 2 * tile_bytes),
           "uncached_host_step_us": round(statistics.median(host_win), 3),
           "device_resident_step_us": round(statistics.median(dev_win), 3),
           "hit_share_by_query_rho": by_rho}
    print(json.dumps(res), flush=True)


def algorithmic_bytes(wl, rec_bytes):
    """Bytes the method must move per step: the summary record of every
    complete page and the K/V rows of every attended token (sink, top-(k-2)
    and the current page's valid tokens; all tokens when J <= k). A quantized
    record counts the pages' byte model, d r/2 + P r + d + 2 (r + P + 1), not
    the library's 16-byte padding."""
    P, k, d, Hkv = wl.page_size, wl.budget_pages, wl.head_dim, wl.num_kv_heads
    if wl.summary_dtype == "i4":
        rec_bytes = d * wl.rank // 2 + P * wl.rank + d + 2 * (wl.rank + P + 1)
    ekv = 2 if wl.kv_dtype == "bf16" else 4
    summary_bytes = kv_bytes = 0
    for T in wl.seq_lens:
        T = int(T)
        J, Jc = -(-T // P), T // P
        summary_bytes += Hkv * Jc * rec_bytes
        A = T if J <= k else (k - 1) * P + (T - (J - 1) * P)
        kv_bytes += Hkv * A * 2 * d * ekv
    return summary_bytes, kv_bytes


PROFILE_CMDS = {
    "stats": ("export TMPDIR=/tmp && cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv \\\n"
              "    -d $OUT/prof_stats -o locks -- python3 -u $R/bench.py --no-cpu-baseline{flags}\n"
              "    (bench.py's default steps and warm-up, so the averages match its timed windows)"),
    "fetch": ("export TMPDIR=/tmp && cd /tmp && timeout -s KILL 240 rocprofv3 --pmc FETCH_SIZE \\\n"
              "    --kernel-include-regex 'locks::|copyBuffer' --output-format csv -d $OUT/prof_fetch "
              "-o fetch \\\n    -- python3 -u $R/bench.py --steps 5 --warmup 2 --no-cpu-baseline "
              "--copy-calibration 256{flags}"),
    "summarize": ("python bench.py{flags} --summarize-profiles $OUT/prof_stats $OUT/prof_fetch "
                  "$OUT/prof_write"),
}

KERNEL_PATTERNS = (("page_score", ("page_score_lds_kernel", "page_score_kernel", "page_score_i4_kernel")),
                   ("select", ("select_kernel",)),
                   ("sparse_decode", ("sparse_decode_kernel",)),
                   ("build", ("build_kernel",)))


def host_pool(t):
    """Pinned host copy of a device pool and the address the GPU reads it at
    (hipHostGetDevicePointer; raises when the memory is not mapped for the
    device, so no kernel ever gets an unmapped address)."""
    import ctypes

    import torch
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
    hip.hipHostGetDevicePointer.restype = ctypes.c_int
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    dptr = ctypes.c_void_p()
    st = hip.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(h.data_ptr()), 0)
    if st != 0 or not dptr.value:
        raise RuntimeError(f"hipHostGetDevicePointer failed ({st})")
    return h, int(dptr.value)


def _clean(name):
    """`void locks::k<...>(locks::Args)` -> `locks::k<...>`"""
    if name.startswith("void "):
        name = name[5:]
    if name.endswith(")") and "(" in name:
        name = name[:name.rindex("(")]
    return name


def _kernel_key(name):
    for key, pats in KERNEL_PATTERNS:
        if any(p in name for p in pats):
            return key
    return None


def summarize_profiles(wl, flags, stats_dir, fetch_dir, write_dir):
    """Write profiles/traffic_<workload>.json, profiles/decode_step_kernels_<workload>.md and
    profiles/memory_traffic_<workload>.md from rocprofv3 CSV output (kernel stats, one
    FETCH_SIZE pass, one WRITE_SIZE pass, each pass ending with plain 256 MiB copies)."""
    import csv
    import glob

    from sparse_kv_page_amd import locks as L
    from sparse_kv_page_amd import synth

    workload = wl.name
    cfg = L.config_for(wl)
    summary_bytes, kv_bytes = algorithmic_bytes(wl, L.locks_summary_record_bytes(cfg))
    alg = {"page_score": summary_bytes, "sparse_decode": kv_bytes}

    def one(pattern):
        hits = sorted(glob.glob(pattern, recursive=True))
        if not hits:
            raise SystemExit(f"no file matches {pattern}")
        return hits[0]

    stats = {}
    with open(one(os.path.join(stats_dir, "**", "*kernel_stats.csv"))) as f:
        for row in csv.DictReader(f):
            if _clean(row["Name"]).startswith("locks::"):
                stats[_clean(row["Name"])] = (int(row["Calls"]), float(row["AverageNs"]) / 1e3,
                                      float(row["MinNs"]) / 1e3, float(row["MaxNs"]) / 1e3)

    def counters(d, counter):
        per_kernel, copies = {}, []
        with open(one(os.path.join(d, "**", "*counter_collection.csv"))) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                v = float(row["Counter_Value"])
                name = _clean(row["Kernel_Name"])
                if "copyBuffer" in name:
                    copies.append((int(row["Dispatch_Id"]), v))
                elif name.startswith("locks::"):
                    per_kernel.setdefault(name, []).append(v)
        # the three calibration copies are the run's last copy dispatches (the
        # copy-bandwidth measurement before them moves larger buffers)
        copies = [v for _, v in sorted(copies)[-3:]]
        return {n: sum(v) / len(v) for n, v in per_kernel.items()}, sum(copies) / len(copies), \
            {n: len(v) for n, v in per_kernel.items()}

    fetch, fetch_copy, calls = counters(fetch_dir, "FETCH_SIZE")
    write, write_copy, _ = counters(write_dir, "WRITE_SIZE")
    copy_kib = 256 * 1024.0
    fs, wsc = copy_kib / fetch_copy, copy_kib / write_copy

    here = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(here, "sparse_kv_page_amd", "csrc")
    rec = {"workload": workload, "fetch_scale": round(fs, 6), "write_scale": round(wsc, 6),
           "calibration": f"3 device copies of 256 MiB (__amd_rocclr_copyBuffer): FETCH_SIZE "
                          f"{fetch_copy:.1f} KiB, WRITE_SIZE {write_copy:.1f} KiB per dispatch",
           "kernels": {}}
    rows_t = []
    for name in sorted(fetch):
        key = _kernel_key(name)
        if key is None or key == "build" or name not in write:
            continue
        traffic = int(round((fetch[name] * fs + write[name] * wsc) * 1024))
        a = alg.get(key)
        avg = next((v[1] for n, v in stats.items() if n == name), None)
        rec["kernels"][key] = {
            "symbol": name, "source_sha1": _sha1([os.path.join(csrc, x) for x in kernel_sources(key, wl)]),
            "fetch_kib": round(fetch[name], 1), "write_kib": round(write[name], 1),
            "hbm_bytes_per_launch": traffic, "algorithmic_bytes_per_launch": a,
            "avg_duration_ns": round(avg * 1e3, 1) if avg else None, "calls": calls[name]}
        rows_t.append(f"| {key} (`{name}`) | {fetch[name]:.1f} | {write[name]:.1f} | {traffic:,} | "
                      f"{a:,} | {traffic / a:.3f} |" if a else
                      f"| {key} (`{name}`) | {fetch[name]:.1f} | {write[name]:.1f} | {traffic:,} | n/a | n/a |")
    os.makedirs(os.path.join(here, "profiles"), exist_ok=True)
    with open(os.path.join(here, "profiles", f"traffic_{workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)

    rows_s = [f"| `{n}` | {c} | {a:.2f} | {lo:.2f} | {hi:.2f} |"
              for n, (c, a, lo, hi) in sorted(stats.items(), key=lambda kv: -kv[1][1])]
    rates = []
    for n, (c, a, lo, hi) in stats.items():
        key = _kernel_key(n)
        if key in alg:
            rates.append(f"{key}: {alg[key]:,} B per launch / {a:.2f} us = "
                         f"{alg[key] / (a * 1e-6) / 1e9:.0f} GB/s ({alg[key] / (a * 1e-6) / 1e9 / HBM_PEAK_GBS:.1%} "
                         f"of 8 TB/s).")
    shape = (f"batch {wl.batch}, {wl.num_q_heads} query / {wl.num_kv_heads} KV heads, d = {wl.head_dim}, "
             f"P = {wl.page_size}, T = {wl.seq_lens[0]}, r = {wl.rank}, k = {wl.budget_pages}, "
             f"{wl.kv_dtype} K/V and {wl.summary_dtype} summaries")
    with open(os.path.join(here, "profiles", f"decode_step_kernels_{workload}.md"), "w") as f:
        f.write(f"# Decode-step kernels, {workload}\n\nWorkload: {shape}; MI355X (gfx950), one GPU, "
                f"ROCm 7.2.\n\nCommand (repository root = `R`, results directory = `OUT`):\n\n    "
                + PROFILE_CMDS["stats"].format(flags=flags).replace("\n", "\n    ") +
                "\n\nThen, without a GPU:\n\n    " + PROFILE_CMDS["summarize"].format(flags=flags) +
                "\n\n| kernel | calls | avg us | min us | max us |\n|---|---|---|---|---|\n" +
                "\n".join(rows_s) + "\n\n" + "\n".join(rates) + "\n")
    with open(os.path.join(here, "profiles", f"memory_traffic_{workload}.md"), "w") as f:
        f.write(f"# Memory traffic of the decode-step kernels, {workload}\n\nSame workload as "
                f"decode_step_kernels_{workload}.md. Two counter passes, one counter each, followed by "
                f"three plain 256 MiB device copies used as the calibration:\n\n    "
                + PROFILE_CMDS["fetch"].format(flags=flags).replace("\n", "\n    ") +
                "\n    (the same with --pmc WRITE_SIZE, -d $OUT/prof_write -o write)\n\n"
                f"Calibration: a 256 MiB copy reads FETCH_SIZE = {fetch_copy:.1f} KiB and WRITE_SIZE = "
                f"{write_copy:.1f} KiB, so FETCH_SIZE is scaled by {fs:.6f} and WRITE_SIZE by {wsc:.6f}.\n\n"
                "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled traffic B/launch | algorithmic B/launch "
                "| ratio |\n|---|---|---|---|---|---|\n" + "\n".join(rows_t) +
                f"\n\ntraffic_{workload}.json holds these figures with the SHA-1 of the kernel sources "
                "they were measured on; bench.py reports them only while the sources match.\n")
    print(json.dumps(rec, indent=1))


# the sources each kernel is compiled from (a measured traffic record is
# reported only while these files are unchanged)
KERNEL_SOURCES = {
    "page_score": ("page_score.hip", "score_lds.h", "common.h", "kernels.h"),
    "page_score_i4": ("page_score_i4.hip", "score_lds.h", "common.h", "kernels.h"),
    "select": ("select.hip", "select_unit.h", "common.h", "kernels.h"),
    "sparse_decode": ("sparse_decode.hip", "decode_split.h", "common.h", "kernels.h"),
}


def kernel_sources(kernel, wl):
    if kernel == "page_score" and wl.summary_dtype == "i4":
        return KERNEL_SOURCES["page_score_i4"]
    return KERNEL_SOURCES.get(kernel)


def _sha1(paths):
    import hashlib
    h = hashlib.sha1()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def roofline(kernel, wl, alg_bytes, avg_us):
    """Roofline record of one kernel: algorithmic bytes per launch over its
    average launch time (HIP events in the timed region), against the HBM
    peak. `traffic` is the measured memory traffic per launch from the
    committed counter record of this workload (FETCH_SIZE + WRITE_SIZE, each
    scaled by a plain copy of known size), and null when that record is
    missing or was taken from a different version of the kernel source."""
    achieved = alg_bytes / (avg_us * 1e-6) / 1e9
    rec = {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
           "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
           "algorithmic_bytes_per_launch": alg_bytes, "avg_launch_us": round(avg_us, 3)}
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"traffic_{wl.name}.json")
    if os.path.exists(path):
        with open(path) as f:
            tr = json.load(f)
        k = tr.get("kernels", {}).get(kernel)
        csrc = os.path.join(here, "sparse_kv_page_amd", "csrc")
        if k and kernel_sources(kernel, wl):
            cur = _sha1([os.path.join(csrc, f) for f in kernel_sources(kernel, wl)])
            if cur == k.get("source_sha1"):
                rec["traffic"] = int(k["hbm_bytes_per_launch"])
                rec["traffic_over_algorithmic"] = round(k["hbm_bytes_per_launch"] / alg_bytes, 4)
    return rec


def selected_kv_footprint(wl, sels, bt):
    """Distinct K/V bytes selected over the rotated query sets (the working
    set that consecutive timed decodes cycle through)."""
    P, d = wl.page_size, wl.head_dim
    e = 2 if wl.kv_dtype == "bf16" else 4
    seen = set()
    bt_c = bt.cpu()
    for sel in sels:
        sc = sel.cpu()
        for b in range(wl.batch):
            for h in range(wl.num_kv_heads):
                for j in sc[b, h].tolist():
                    if j >= 0:
                        seen.add((int(bt_c[b, j]), h))
    return len(seen) * P * 2 * d * e


class ThrottleMonitor:
    """Reads the GPU's accumulated violation counters (thermal, power, VR,
    HBM thermal residency) from the amdsmi metrics table; a window is
    throttled when any of them grew while it ran. Reports itself unavailable
    when amdsmi cannot reach the GPU. The metrics table is read directly
    (about 0.6 ms) rather than through the violation-status call, which
    samples for about 100 ms: an idle GPU that long lowers its clocks, and the
    next timed window started several percent slow."""
    KEYS = ("acc_prochot_thrm", "acc_ppt_pwr", "acc_socket_thrm", "acc_vr_thrm", "acc_hbm_thrm")
    # metrics-table field of each key
    FIELDS = {"acc_prochot_thrm": "prochot_residency_acc", "acc_ppt_pwr": "ppt_residency_acc",
              "acc_socket_thrm": "socket_thm_residency_acc", "acc_vr_thrm": "vr_thm_residency_acc",
              "acc_hbm_thrm": "hbm_thm_residency_acc", "acc_counter": "accumulation_counter"}

    def __init__(self):
        self.h = None
        self.err = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if not handles:
                raise RuntimeError("no GPU handle")
            self.h = handles[0]
            self.smi = amdsmi
            m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
            missing = [f for f in self.FIELDS.values() if f not in m]
            if missing:
                raise RuntimeError(f"metrics table lacks {missing}")
        except Exception as ex:  # noqa: BLE001 - monitoring only
            self.h = None
            self.err = f"{type(ex).__name__}: {ex}"[:200]

    def read(self):
        if self.h is None:
            return None
        try:
            m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
            return {k: m.get(f) for k, f in self.FIELDS.items()}
        except Exception as ex:  # noqa: BLE001
            self.err = f"{type(ex).__name__}: {ex}"[:200]
            return None

    def read_sampled(self):
        """The same counters through amdsmi's violation-status call (which
        samples for about 100 ms); only outside timed windows."""
        if self.h is None:
            return None
        try:
            v = self.smi.amdsmi_get_violation_status(self.h)
            return {k: v.get(k) for k in self.KEYS + ("acc_counter",)}
        except Exception as ex:  # noqa: BLE001
            self.err = f"{type(ex).__name__}: {ex}"[:200]
            return None

    def delta(self, a, b):
        if a is None or b is None:
            return {"available": False, "reason": self.err}
        out = {"available": True}
        grew = False
        for k in self.KEYS + ("acc_counter",):
            x, y = a.get(k), b.get(k)
            dv = (y - x) if isinstance(x, int) and isinstance(y, int) else None
            out[k] = dv
            if k != "acc_counter" and dv:
                grew = True
        out["throttled"] = grew
        return out


def copy_bandwidth(dev, mib=1024, reps=5):
    """Device-to-device copy of `mib` MiB (read + write bytes over time), the
    best of `reps` copies: the bandwidth this machine delivers to a plain stream."""
    import torch
    src = torch.ones(mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del src, dst
    return {"bytes_moved": 2 * (mib << 20), "GBps": round(2 * (mib << 20) / (best * 1e-3) / 1e9, 1),
            "kernel": "torch copy_ (device to device)"}


def host_cpus():
    """CPUs this process may run on: the affinity mask, cut to the cgroup CPU
    quota when one is set; and the CPU model."""
    n = len(os.sched_getaffinity(0))
    quota = None
    try:
        q, per = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if q != "max":
            quota = float(q) / float(per)
    except (OSError, ValueError):
        try:
            q = int(open("/sys/fs/cgroup/cpu/cpu.cfs_quota_us").read())
            per = int(open("/sys/fs/cgroup/cpu/cpu.cfs_period_us").read())
            if q > 0:
                quota = q / per
        except (OSError, ValueError):
            pass
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    usable = n if quota is None else max(1, min(n, int(math.ceil(quota))))
    return usable, {"affinity_cpus": n, "cgroup_cpu_quota": quota, "os_cpu_count": os.cpu_count(),
                    "cpu_model": model}


# the CPU share of one GPU on the machines this runs on: worker pools stay within it
CPU_SHARE_PER_GPU = 16


def cpu_baseline(wl, cfg, data, seconds, step_bytes):
    """The fp64 oracle (score -> combine -> select -> attend, test
    infrastructure, untuned) on a bounded sample of the same step, with
    synthetic summary records of the same shape, timed with every usable host
    CPU and with one thread: each leg three runs of about seconds / 6, median
    reported, scaled to one full step."""
    import torch

    import oracle
    from sparse_kv_page_amd import synth

    usable, info = host_cpus()
    threads_all = max(1, min(usable, CPU_SHARE_PER_GPU))

    def sample(nseq):
        sub = wl.with_(batch=nseq, seq_lens=wl.seq_lens[:nseq])
        bt = data["block_table"][:nseq].cpu()
        used = torch.unique(bt.reshape(-1)).long()
        remap = torch.full((wl.num_blocks,), -1, dtype=torch.long)
        remap[used] = torch.arange(used.numel())
        bt_local = remap[bt.long()].numpy()
        to32 = lambda t: t.to("cpu", torch.float32).numpy()
        kp = to32(data["k_pool"][used.to(data["k_pool"].device)])
        vp = to32(data["v_pool"][used.to(data["v_pool"].device)])
        # records indexed by the local block ids; quantized records are
        # dequantized by the oracle inside the timed loop
        if wl.summary_dtype == "i4":
            codes = synth.random_i4_codes(sub.with_(extra_blocks=0), seed=1, device="cpu")
            codes = {kk: v.reshape((-1,) + tuple(v.shape[2:])).numpy() for kk, v in codes.items()}
            shape = (used.numel(), wl.num_kv_heads)

            def summaries():
                m, v, c = oracle.dequantize_summaries(codes)
                return tuple(x.reshape(shape + x.shape[1:]) for x in (m, v, c))
        else:
            recs = [x.double().numpy() for x in synth.random_summaries(sub.with_(extra_blocks=0), seed=1,
                                                                        device="cpu")]

            def summaries():
                return recs
        q = data["q"][:nseq].to("cpu", torch.float64).numpy()
        return sub, q, kp, vp, bt_local, summaries

    def leg(nseq, units, threads, budget_s):
        sub, q, kp, vp, bt_local, summaries = sample(nseq)
        run = lambda: oracle.decode_step(q, *summaries(), kp, vp, bt_local, list(sub.seq_lens), wl.page_size,
                                         wl.budget_pages, wl.softmax_scale, units=units, threads=threads)
        run()  # warm (loads the library)
        per_unit = []
        for _ in range(3):
            reps, t0 = 0, time.perf_counter()
            while True:
                run()
                reps += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            per_unit.append((time.perf_counter() - t0) / reps / len(units))
        n_units = wl.batch * wl.num_kv_heads
        runs_us = [round(x * n_units * 1e6, 1) for x in per_unit]
        return statistics.median(runs_us), runs_us

    nseq = min(2, wl.batch)
    all_units = [(b, h) for b in range(nseq) for h in range(wl.num_kv_heads)]
    one_units = all_units[:2]
    v_all, runs_all = leg(nseq, all_units, threads_all, seconds / 6)
    v_one, runs_one = leg(nseq, one_units, 1, seconds / 6)
    return {"value": v_all, "unit": "us", "cores": threads_all, "kind": "oracle",
            "sample": f"{len(all_units)} of {wl.batch * wl.num_kv_heads} (sequence, KV head) units "
                      f"(score+combine+select+attend, fp64), scaled to the whole step; median of 3 runs",
            "runs_us": runs_all, "GBps_effective": round(step_bytes / (v_all * 1e-6) / 1e9, 2),
            "one_thread": {"value": v_one, "unit": "us", "runs_us": runs_one,
                           "sample": f"{len(one_units)} units, scaled to the whole step"},
            "host": dict(info, usable_cpus=usable, thread_cap=CPU_SHARE_PER_GPU)}


if __name__ == "__main__":
    main()

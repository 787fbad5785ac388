"""Throughput of the fused block-sparse paged decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--index bf16|fp8]

One step = metadata -> index score + pooling -> top-k + page-16 table + ctx ->
sparse paged attention + split merge (msa_sparse_decode) over one batch of the
named synthetic workload (default: 8 requests x 1 row, L ~ U{8192..32768},
top-k 16, 16 query heads, bf16; --index fp8 stores the index keys as e4m3fn
codes with per-token scales). The step's inputs live in HBM; several copies
of the caches at different addresses are cycled so that no step finds the
previous step's data in the 256 MB Infinity Cache. Steps are replayed from a
HIP graph holding one step per copy. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-decode query rows/sec + achieved HBM GB/s (% of MI355X peak)"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 MFMA
WORKLOAD_DESC = {
    "tiny": "tiny decode: 1 request x 1 row, L=2048, top-k 4, 8 q heads / 1 kv head, bf16",
    "bf16_batch": "bf16 decode batch: 8 requests x 1 row, L~U{8192..32768}, permuted pages, top-k 16, "
                  "16 q heads / 1 kv head, head dim 128, index dim 128, bf16",
    "spec_decode": "speculative decode: 4 requests x 4 rows, L=65536, top-k 32, 16 q heads, bf16",
    "fp8_kv": "fp8 kv: 11 requests x 1 row, L~U{32768..131072}, e4m3fn K/V + per-token-head scales, top-k 64",
    "mixed_prefill": "mixed: 6 decode rows (L=16384) + 2x4096 prefill rows on 28672 context, top-k 32",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="bf16_batch", choices=sorted(WORKLOAD_DESC))
    p.add_argument("--index", default="bf16", choices=("bf16", "fp8"),
                   help="index cache: bf16 keys, or e4m3fn codes with one fp32 scale per token")
    p.add_argument("--copies", type=int, default=0, help="cache copies cycled (0: enough for 768 MB)")
    p.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying graphs")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--counters", action="store_true",
                   help="counter pass: 8 plain copies of 256 MiB, then 8 index-score launches, no timing")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="turn two rocprofv3 --pmc outputs (FETCH_SIZE, WRITE_SIZE) of --counters into "
                        "the traffic summary under profiles/")
    p.add_argument("--summarize-trace", metavar="TRACE_DIR",
                   help="turn a rocprofv3 --kernel-trace --stats csv output into a summary under profiles/")
    p.add_argument("--summarize-mfma", metavar="PMC_DIR",
                   help="turn a rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE output "
                        "into a per-kernel MFMA-utilisation summary under profiles/")
    return p.parse_args()


COPY_BYTES = 256 << 20
TRAFFIC_FILE = "index_score_traffic_{}.json"


def algorithmic_bytes(b, ctx):
    """Minimum HBM bytes of one step and of its index-score launch.
    index-K: every visible token of every request once (128 bf16 = 256 B, or
    128 e4m3fn codes + a 4-byte scale = 132 B);
    K/V: each row's ctx tokens (K and V rows of 128 elements, plus per-token
    scales); q/out/index_q once; scores, tables, ctx and metadata."""
    import numpy as np
    N, hq, ld_s, topk = b.num_rows, b.num_q_heads, b.ld_s, b.topk
    elt = 2 if b.kv_dtype == 0 else 1
    idx_k = int(b.seq_lens.astype(np.int64).sum()) * (256 if b.index_scale is None else 132)
    score_launch = idx_k + N * 256 + N * ld_s * 4
    kv_tok = 2 * 128 * elt + (8 if b.scale_mode == 2 else 0)
    kv = int(np.asarray(ctx, dtype=np.int64).sum()) * kv_tok
    qo = N * hq * 128 * 2 * 2
    small = N * ld_s * 4 * 2 + N * 8 * topk * 4 + N * 4 + N * topk * 4 + b.num_reqs * 4 * 6 + N * 8
    return {"step": idx_k + N * 256 + kv + qo + small, "score": score_launch, "attn": kv + qo + N * 8 * topk * 4,
            "kv": kv}


def unique_kv_bytes(b, table, ctx):
    """K/V bytes of a step when each sub-page that any row of a request
    attends is read once for the request (the rows' page-16 tables give the
    sub-pages: the first ceil(ctx/16) entries of each row), the K/V term of
    the step's minimum traffic once rows of one request share blocks."""
    import numpy as np
    elt = 2 if b.kv_dtype == 0 else 1
    kv_tok = 2 * 128 * elt + (8 if b.scale_mode == 2 else 0)
    cu = np.concatenate([[0], np.cumsum(b.query_lens.astype(np.int64))])
    total = 0
    for r in range(b.num_reqs):
        parts = [table[n, :(int(ctx[n]) + 15) // 16] for n in range(cu[r], cu[r + 1])]
        if parts:
            total += int(np.unique(np.concatenate(parts)).size) * 16 * kv_tok
    return total


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(b, rows, budget_s=10.0):
    """The oracle as it stands, single-threaded, on `rows` of the workload,
    repeated until about budget_s seconds of CPU work."""
    from threadpoolctl import threadpool_limits

    from oracle import msa_oracle as O
    passes = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            O.decode_step(b, rows=rows)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= budget_s:
                break
    return {"value": passes * len(rows) / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} passes over {len(rows)} of {b.num_rows} rows of the {b.name} workload, "
                      f"full step (metadata, scores, pooling, selection, table, attention), {dt:.1f} s, {cpu_model()}"}


_PAR_BATCH = None  # the batch the parallel oracle workers read (inherited through fork)


def _oracle_row(n):
    from oracle import msa_oracle as O
    O.decode_step(_PAR_BATCH, rows=[n])
    return n


def _single_thread_worker():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def cpu_baseline_parallel(b, rows, budget_s=10.0):
    """The oracle as it stands, one row per task over a pool of single-thread
    worker processes (one per host core the process may use, at most one per
    row), repeated until about budget_s seconds. Runs before the GPU is
    touched: the workers are forked from this process."""
    import concurrent.futures
    import multiprocessing
    global _PAR_BATCH
    _PAR_BATCH = b
    cores = max(1, min(len(rows), len(os.sched_getaffinity(0)), 16))
    ctx = multiprocessing.get_context("fork")
    with concurrent.futures.ProcessPoolExecutor(cores, mp_context=ctx, initializer=_single_thread_worker) as ex:
        list(ex.map(_oracle_row, rows))  # workers up and warm
        passes = 0
        t0 = time.perf_counter()
        while True:
            list(ex.map(_oracle_row, rows))
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= budget_s:
                break
    _PAR_BATCH = None
    return {"value": passes * len(rows) / dt, "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": f"{passes} passes over {len(rows)} of {b.num_rows} rows of the {b.name} workload, one row per "
                      f"task on {cores} single-thread worker processes, full step per row, {dt:.1f} s, {cpu_model()}"}


def time_insert(msa, torch, tokens=8192, copies=32, reps=32):
    """msa_cache_insert of a prefill chunk (two sequences of 4096 new tokens, the
    mixed workload's prefill shape) into fp8 e4m3fn caches with per-token-head
    scales, index-K included: per-launch time over back-to-back launches in one
    graph, cycling `copies` sets of inputs and caches (>= 256 MB in all, so no
    launch finds its data in the Infinity Cache). Algorithmic bytes per token:
    K, V and index-K rows read (3 x 256 B) + the slot (4 B); fp8 K and V (2 x 128
    B), their scales (2 x 4 B) and the index-K row (256 B) written."""
    dev = "cuda"
    pages = tokens // 128
    g = torch.Generator(device="cpu").manual_seed(11)
    sets = []
    for c in range(copies):
        k_new = (torch.randn((tokens, 1, 128), generator=g) * 2).to(torch.bfloat16).to(dev)
        v_new = (torch.randn((tokens, 1, 128), generator=g) * 2).to(torch.bfloat16).to(dev)
        i_new = torch.randn((tokens, 128), generator=g).to(torch.bfloat16).to(dev)
        perm = torch.randperm(pages, generator=g)
        t = torch.arange(tokens)
        slots = (perm[t // 128] * 128 + t % 128).to(torch.int32).to(dev)
        kc = torch.zeros((pages * 8, 1, 2048), dtype=torch.uint8, device=dev)
        vc = torch.zeros((pages * 8, 1, 2048), dtype=torch.uint8, device=dev)
        ks = torch.ones((pages * 8, 16, 1), dtype=torch.float32, device=dev)
        vs = torch.ones((pages * 8, 16, 1), dtype=torch.float32, device=dev)
        ik = torch.zeros((pages, 128 * 128), dtype=torch.int16, device=dev)
        kv = msa.make_kv(kc, vc, 1, 2, pages, ks, vs)
        sets.append((slots, k_new, v_new, i_new, ik, kv, kc, vc, ks, vs))
    stream = torch.cuda.current_stream()
    gs = torch.cuda.Stream()
    gs.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gs):
        for st in sets:
            msa.msa_cache_insert(tokens, st[0], st[1], st[2], st[5], st[3], st[4])
        with torch.cuda.graph(graph, stream=gs):
            for i in range(reps):
                st = sets[i % copies]
                msa.msa_cache_insert(tokens, st[0], st[1], st[2], st[5], st[3], st[4])
    stream.wait_stream(gs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    runs = []
    for _ in range(5):
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        runs.append(e0.elapsed_time(e1) * 1e3 / reps)
    us = sorted(runs)[len(runs) // 2]
    nbytes = tokens * (3 * 256 + 4 + 2 * 128 + 2 * 4 + 256)
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "msa_insert_kernel (msa_cache_insert)", "tokens": tokens,
            "kv": "fp8 e4m3fn, per-token-head scales, index-K written", "us_per_launch": us,
            "tokens_per_s": tokens / (us * 1e-6), "algorithmic_bytes": nbytes, "achieved": gbps,
            "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": gbps / PEAK_HBM_GBPS}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the decode path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    if args.summarize_counters:
        summarize_counters(args.workload, args.index, *args.summarize_counters)
        return
    if args.summarize_trace:
        summarize_trace(args.workload, args.index, args.summarize_trace)
        return
    if args.summarize_mfma:
        summarize_mfma(args.workload, args.index, args.summarize_mfma)
        return

    import numpy as np
    import torch

    import block_sparse_paged_msa_amd as msa
    import msa_synth as syn

    idx_fp8 = args.index == "fp8"
    b = syn.config(args.workload, index_dtype=syn.INDEX_FP8 if idx_fp8 else syn.INDEX_BF16)
    cpu_par = None
    if not args.no_cpu_baseline:  # before the GPU is touched (the pool forks this process)
        print("[bench] cpu baseline, all cores (oracle) ...", file=sys.stderr, flush=True)
        cpu_par = cpu_baseline_parallel(b, list(range(min(b.num_rows, 8))))
    torch.cuda.set_device(0)
    msa.load()
    N, R, P, hq, topk, ld_s = b.num_rows, b.num_reqs, b.num_pages, b.num_q_heads, b.topk, b.ld_s
    per_copy = b.index_k.nbytes + b.k_cache.nbytes + b.v_cache.nbytes + (b.index_scale.nbytes if idx_fp8 else 0)
    copies = args.copies or max(2, math.ceil(768e6 / per_copy))
    dev = "cuda"

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()) if a.dtype == np.uint16 \
            else torch.from_numpy(np.ascontiguousarray(a).copy())

    # cache pools holding `copies` replicas of the pages, each copy on its own pages
    def pool(a):
        one = t16(a).to(dev)
        out = torch.empty((copies,) + tuple(one.shape), dtype=one.dtype, device=dev)
        out[:] = one
        return out.view((copies * one.shape[0],) + tuple(one.shape[1:]))

    index_k = pool(b.index_k)
    index_scale = pool(b.index_scale) if idx_fp8 else None
    k_cache = pool(b.k_cache)
    v_cache = pool(b.v_cache)
    k_scale = v_scale = None
    if b.scale_mode == syn.SCALE_PER_TOKEN_HEAD:
        k_scale, v_scale = pool(b.k_scale), pool(b.v_scale)
    elif b.scale_mode == syn.SCALE_SCALAR:
        k_scale, v_scale = t16(b.k_scale).to(dev), t16(b.v_scale).to(dev)
    index_q = t16(b.index_q).to(dev)
    q = t16(b.q).to(dev)
    seq_lens = torch.from_numpy(b.seq_lens).to(dev)
    query_lens = torch.from_numpy(b.query_lens).to(dev)
    kv = msa.make_kv(k_cache, v_cache, b.kv_dtype, b.scale_mode, copies * P, k_scale, v_scale)

    i32 = dict(dtype=torch.int32, device=dev)
    batches, keep = [], []
    for c in range(copies):
        bt = torch.from_numpy(b.block_table + c * P).to(dev)
        meta = [torch.empty(R + 1, **i32) for _ in range(4)] + [torch.empty(N, **i32) for _ in range(2)]
        keep += [bt] + meta
        batches.append(msa.make_batch(seq_lens, query_lens, bt, *meta, R, N, b.max_seq_len, copies * P))

    out = torch.empty((N, hq, 128), dtype=torch.int16, device=dev)
    table = torch.empty((N, 8 * topk), **i32)
    ctx = torch.empty((N,), **i32)
    scores = torch.empty((N, ld_s), dtype=torch.float32, device=dev)
    wsb = msa.msa_decode_workspace_bytes(N, b.max_seq_len, hq, topk, 0)  # prefill-sized: block-major path
    ws = torch.empty((wsb,), dtype=torch.uint8, device=dev)

    def step(c):
        if idx_fp8:
            msa.msa_sparse_decode_ex(batches[c], index_q, index_k, index_scale, q, hq, kv, topk, b.sm_scale, None,
                                     out, None, table, ctx, None, scores, ld_s, ws, wsb)
        else:
            msa.msa_sparse_decode(batches[c], index_q, index_k, q, hq, kv, topk, b.sm_scale, out, table, ctx,
                                  None, scores, ld_s, ws, wsb)

    def score(c):
        msa.msa_index_score_ex(batches[c], index_q, index_k, index_scale, scores, ld_s)

    for c in range(copies):
        step(c)
    torch.cuda.synchronize()
    if args.counters:
        # counter pass: plain copies of known size, then the dominant kernel
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(8):
            torch.mul(src, 1, out=dst)   # an elementwise kernel: reads and writes COPY_BYTES
        torch.cuda.synchronize()
        for i in range(8):
            score(i % copies)
        torch.cuda.synchronize()
        print(json.dumps({"counters_pass": args.workload, "copy_bytes": COPY_BYTES,
                          "score_algorithmic_bytes": algorithmic_bytes(b, ctx.cpu().numpy())["score"]}))
        return
    ctx_host = ctx.cpu().numpy()
    nbytes = algorithmic_bytes(b, ctx_host)
    kv_unique = unique_kv_bytes(b, table.cpu().numpy(), ctx_host)

    if args.eager:
        def run_steps(k0, k):
            for i in range(k0, k0 + k):
                step(i % copies)
    else:
        # one graph holding one step per cache copy, plus one graph per copy for
        # a remainder, so that exactly the requested number of steps is replayed
        graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            g_all = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_all, stream=s):
                for c in range(copies):
                    step(c)
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    step(c)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()

        def run_steps(k0, k):
            full, rem = divmod(k, copies)
            for _ in range(full):
                g_all.replay()
            for i in range(rem):
                graphs[i].replay()

    run_steps(0, args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(0, args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec = (t1 - t0) / args.steps
    print(f"[bench] {args.workload}: {sec * 1e6:.2f} us/step over {args.steps} steps, {copies} copies",
          file=sys.stderr, flush=True)

    # Per-step latency distribution: single steps, each bracketed by HIP
    # events on the launching stream, cycling the cache copies (a replay of a
    # one-step graph, or the eager launches); the first replays are warm-up.
    lat_stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(100)]
    for i in range(10 + len(ev)):
        c = i % copies
        if i >= 10:
            ev[i - 10][0].record(lat_stream)
        if args.eager:
            step(c)
        else:
            graphs[c].replay()
        if i >= 10:
            ev[i - 10][1].record(lat_stream)
    torch.cuda.synchronize()
    lat = np.sort(np.array([a.elapsed_time(b_) * 1e3 for a, b_ in ev]))
    step_lat = {"p10_us": float(np.percentile(lat, 10)), "p50_us": float(np.percentile(lat, 50)),
                "p90_us": float(np.percentile(lat, 90)), "samples": int(lat.size),
                "note": "each step a separate replay between two events: includes the per-replay launch "
                        "overhead that back-to-back steps (ms_per_step) hide"}

    # Dominant kernel: back-to-back msa_index_score launches (cycling the cache
    # copies) captured in one graph and bracketed by HIP events on the
    # launching stream, so the per-launch figure is the kernel's own duration
    # plus the small gap between graph nodes.
    reps = 32
    stream = torch.cuda.current_stream()
    gs = torch.cuda.Stream()
    gs.wait_stream(stream)
    g_score = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gs):
        score(0)
        with torch.cuda.graph(g_score, stream=gs):
            for i in range(reps):
                score(i % copies)
    stream.wait_stream(gs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_score_runs = []
    for _ in range(5):
        e0.record(stream)
        g_score.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        t_score_runs.append(e0.elapsed_time(e1) * 1e3 / reps)
    t_score = sorted(t_score_runs)[len(t_score_runs) // 2]

    score_gbps = nbytes["score"] / (t_score * 1e-6) / 1e9
    traffic = None
    tpath = os.path.join(ROOT, "profiles", TRAFFIC_FILE.format(tag(args.workload, args.index)))
    if os.path.exists(tpath):
        try:
            tj = json.load(open(tpath))
            if tj.get("kernel_source_hash") == source_hash():
                traffic = tj.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None

    res = {
        "metric": METRIC,
        "value": N / sec,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if b.kv_dtype == 0 else "fp8-kv/bf16",
        "data": "synthetic (seeded splitmix64 N(0,1) values, random page permutation)",
        "config": {"workload": WORKLOAD_DESC[args.workload] + (
                       ", fp8 e4m3fn index keys + per-token scales" if idx_fp8 else ""),
                   "requests": R, "rows": N, "top_k": topk,
                   "q_heads": hq, "kv_heads": 1, "head_dim": 128, "seq_lens_sum": int(b.seq_lens.sum()),
                   "cache_copies_cycled": copies, "graphs": not args.eager},
        "step_latency": step_lat,
        "step_hbm_gbps": nbytes["step"] / sec / 1e9,
        "step_hbm_frac": nbytes["step"] / sec / 1e9 / PEAK_HBM_GBPS,
        "step_algorithmic_bytes": nbytes["step"],
        # the same with each request's attended K/V counted once (rows of one
        # request that select the same blocks share them)
        "step_unique_bytes": nbytes["step"] - nbytes["kv"] + kv_unique,
        "step_unique_hbm_frac": (nbytes["step"] - nbytes["kv"] + kv_unique) / sec / 1e9 / PEAK_HBM_GBPS,
        "roofline": {"kernel": "msa_score_kernel (msa_index_score)", "bound": "hbm", "achieved": score_gbps,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": score_gbps / PEAK_HBM_GBPS,
                     "traffic": traffic, "algorithmic_bytes": nbytes["score"], "avg_launch_us": t_score},
    }
    if (b.query_lens > 64).any():
        # requests of more than 64 rows are scored by the MFMA tile kernel:
        # 2 * 128 flops per (row, visible token) over every row of the launch
        pos = b.seq_lens.astype(np.int64) - b.query_lens.astype(np.int64)
        vis = sum(int(ql) * int(p0) + int(ql) * (int(ql) + 1) // 2 for p0, ql in zip(pos, b.query_lens))
        tflops = 2 * 128 * vis / (t_score * 1e-6) / 1e12
        res["score_mfma"] = {"kernels": "msa_score_kernel + msa_score_tile_kernel (one msa_index_score call)",
                             "bound": "mfma", "algorithmic_flop": 2 * 128 * vis, "us_per_call": t_score,
                             "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                             "frac": tflops / PEAK_BF16_TFLOPS}
    res["cache_insert"] = time_insert(msa, torch)

    # the same step through msa_sparse_decode_ex: LSE written, per-head sinks
    # applied; both variants timed here the same way (one graph of `copies`
    # steps, replayed)
    sinks = torch.linspace(-1.0, 2.0, hq, device=dev, dtype=torch.float32)
    lse = torch.empty((N, hq), dtype=torch.float32, device=dev)

    def step_lse(c):
        msa.msa_sparse_decode_ex(batches[c], index_q, index_k, index_scale, q, hq, kv, topk, b.sm_scale, sinks,
                                 out, lse, table, ctx, None, scores, ld_s, ws, wsb)

    def graph_us_per_step(fn):
        gs2 = torch.cuda.Stream()
        gs2.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs2):
            with torch.cuda.graph(g, stream=gs2):
                for c in range(copies):
                    fn(c)
        stream.wait_stream(gs2)
        torch.cuda.synchronize()
        reps_g = max(1, 192 // copies)
        runs = []
        for _ in range(5):
            e0.record(stream)
            for _ in range(reps_g):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            runs.append(e0.elapsed_time(e1) * 1e3 / (reps_g * copies))
        return sorted(runs)[len(runs) // 2]

    res["lse_sinks"] = {"entry": "msa_sparse_decode_ex", "us_per_step": graph_us_per_step(step_lse),
                        "plain_us_per_step": graph_us_per_step(step), "rows": N, "q_heads": hq}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(b, list(range(min(N, 8))))
        res["cpu_baseline_all_cores"] = cpu_par
    print(json.dumps(res), flush=True)


def _counter_rows(d):
    """(kernel name, counter name, value) rows of a rocprofv3 --pmc csv output."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for rec in csv.DictReader(fh):
                rows.append((rec.get("Kernel_Name", ""), rec.get("Counter_Name", ""),
                             float(rec.get("Counter_Value", "nan"))))
    return rows


PMC_CMD = ("rocprofv3 --pmc {counter} --output-format csv -d <out> -o run -- "
           "python3 -u bench.py --workload {workload}{index} --counters")
TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o bench -- "
             "python3 -u bench.py --workload {workload}{index} --steps 50 --warmup 10 --no-cpu-baseline")


def tag(workload, index):
    """File-name tag of a workload (and of its fp8-index variant)."""
    return workload if index == "bf16" else f"{workload}_fp8index"


def _index_flag(index):
    return "" if index == "bf16" else f" --index {index}"


def _short(name):
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return name.split("(")[0]


def summarize_counters(workload, index, fetch_dir, write_dir):
    """Scale every kernel's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what
    the same counter reads for the calibration kernel of the --counters pass
    (an elementwise multiply that reads and writes COPY_BYTES bytes). Writes
    the index-score kernel's traffic for bench.py and a per-kernel table."""
    import statistics
    name = tag(workload, index)
    out = {"workload": name, "kernel": "msa_score_kernel", "copy_bytes": COPY_BYTES,
           "kernel_source_hash": source_hash()}
    table = {}
    total = 0.0
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r[1] == counter]
        copy = [v for k, _, v in rows if "MulFunctor" in k]
        if not copy:
            raise SystemExit(f"no calibration-kernel {counter} rows in {d}")
        c_kib = statistics.median(copy)
        factor = COPY_BYTES / (c_kib * 1024.0)
        per = {}
        for k, _, v in rows:
            if "msa_" in k:
                per.setdefault(_short(k), []).append(v)
        for k, vals in per.items():
            table.setdefault(k, {})[counter] = statistics.median(vals) * 1024.0 * factor
        score_key = next(k for k in per if k.startswith("msa_score_kernel"))
        s_kib = statistics.median(per[score_key])
        out[counter] = {"calibration_kib_per_dispatch": c_kib, "score_kib_per_dispatch": s_kib,
                        "scale_factor": factor, "score_bytes": s_kib * 1024.0 * factor}
        total += s_kib * 1024.0 * factor
    out["bytes_per_launch"] = total
    prof = os.path.join(ROOT, "profiles")
    with open(os.path.join(prof, TRAFFIC_FILE.format(name)), "w") as fh:
        json.dump(out, fh, indent=1)
    fl = _index_flag(index)
    lines = [f"# HBM traffic per dispatch, {name} workload", "",
             "Commands (one counter per run, outputs in <out>):", "",
             "    " + PMC_CMD.format(counter="FETCH_SIZE", workload=workload, index=fl),
             "    " + PMC_CMD.format(counter="WRITE_SIZE", workload=workload, index=fl),
             "    python3 bench.py --workload {}{} --summarize-counters <fetch-out> <write-out>".format(workload, fl),
             "",
             "Calibration: an elementwise multiply over {} MiB reads FETCH_SIZE {:.0f} KiB and WRITE_SIZE "
             "{:.0f} KiB per dispatch, so the counters are scaled by {:.3f} (fetch) and {:.3f} (write)."
             .format(COPY_BYTES >> 20, out["FETCH_SIZE"]["calibration_kib_per_dispatch"],
                     out["WRITE_SIZE"]["calibration_kib_per_dispatch"], out["FETCH_SIZE"]["scale_factor"],
                     out["WRITE_SIZE"]["scale_factor"]), "",
             "| kernel | fetched MB | written MB |", "|---|---|---|"]
    for k, v in sorted(table.items()):
        lines.append(f"| {k} | {v.get('FETCH_SIZE', float('nan')) / 1e6:.3f} | {v.get('WRITE_SIZE', float('nan')) / 1e6:.3f} |")
    lines += ["", f"Kernel source hash (msa_score.hip + msa_internal.h): {out['kernel_source_hash']}"]
    with open(os.path.join(prof, f"counters_{name}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(json.dumps(out))


def summarize_trace(workload, index, trace_dir):
    """Per-kernel duration table from a rocprofv3 --stats csv output."""
    import csv
    import glob
    f = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not f:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    name = tag(workload, index)
    lines = [f"# Kernel durations, {name} workload", "", "Command:", "",
             "    " + TRACE_CMD.format(workload=workload, index=_index_flag(index)), "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    with open(f[0]) as fh:
        for rec in csv.DictReader(fh):
            if "msa_" not in rec["Name"]:
                continue
            lines.append(f"| {_short(rec['Name'])} | {rec['Calls']} | {float(rec['AverageNs']) / 1e3:.2f} | "
                         f"{float(rec['MinNs']) / 1e3:.2f} | {float(rec['MaxNs']) / 1e3:.2f} |")
    with open(os.path.join(ROOT, "profiles", f"kernel_trace_{name}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


MFMA_CMD = ("rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv "
            "-d <out> -o run -- python3 -u bench.py --workload {workload}{index} --steps 3 --warmup 1 --eager "
            "--no-cpu-baseline")
NUM_XCD, NUM_SIMD = 8, 1024  # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def summarize_mfma(workload, index, pmc_dir):
    """Per-kernel MFMA busy fraction from one --pmc pass: the MFMA busy cycles
    summed over every SIMD, divided by the kernel's active cycles (GRBM_GUI_ACTIVE
    is summed over the 8 XCDs, so it is divided by 8) times the 1024 SIMDs."""
    import statistics
    name = tag(workload, index)
    per = {}
    for k, c, v in _counter_rows(pmc_dir):
        if "msa_" in k:
            per.setdefault(_short(k), {}).setdefault(c, []).append(v)
    lines = [f"# MFMA utilisation per kernel, {name} workload", "", "Command:", "",
             "    " + MFMA_CMD.format(workload=workload, index=_index_flag(index)),
             f"    python3 bench.py --workload {workload}{_index_flag(index)} --summarize-mfma <out>", "",
             "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs), medians over "
             "dispatches; active us = GRBM_GUI_ACTIVE / 8 at 2.4 GHz.", "",
             "| kernel | dispatches | active us | MFMA busy |", "|---|---|---|---|"]
    for k, cs in sorted(per.items()):
        if "GRBM_GUI_ACTIVE" not in cs or "SQ_VALU_MFMA_BUSY_CYCLES" not in cs:
            continue
        act = statistics.median(cs["GRBM_GUI_ACTIVE"]) / NUM_XCD
        busy = statistics.median(cs["SQ_VALU_MFMA_BUSY_CYCLES"])
        lines.append(f"| {k} | {len(cs['GRBM_GUI_ACTIVE'])} | {act / 2400:.1f} | "
                     f"{100.0 * busy / max(act * NUM_SIMD, 1.0):.1f}% |")
    with open(os.path.join(ROOT, "profiles", f"mfma_{name}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


def source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("msa_score.hip", "msa_internal.h"):
        with open(os.path.join(ROOT, "block_sparse_paged_msa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()

"""Throughput of the fused block-sparse paged decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = metadata -> index score + pooling -> top-k + page-16 table + ctx ->
sparse paged attention + split merge (msa_sparse_decode) over one batch of the
named synthetic workload (default: 8 requests x 1 row, L ~ U{8192..32768},
top-k 16, 16 query heads, bf16). The step's inputs live in HBM; several copies
of the caches at different addresses are cycled so that no step finds the
previous step's data in the 256 MB Infinity Cache. Steps are replayed from HIP
graphs (one per copy). Prints one JSON line.
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
    p.add_argument("--copies", type=int, default=0, help="cache copies cycled (0: enough for 768 MB)")
    p.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying graphs")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"))
    return p.parse_args()


def algorithmic_bytes(b, ctx):
    """Minimum HBM bytes of one step and of its index-score launch.
    index-K: every visible token of every request once (128 bf16 = 256 B);
    K/V: each row's ctx tokens (K and V rows of 128 elements, plus per-token
    scales); q/out/index_q once; scores, tables, ctx and metadata."""
    import numpy as np
    N, hq, ld_s, topk = b.num_rows, b.num_q_heads, b.ld_s, b.topk
    elt = 2 if b.kv_dtype == 0 else 1
    idx_k = int(b.seq_lens.astype(np.int64).sum()) * 256
    score_launch = idx_k + N * 256 + N * ld_s * 4
    kv_tok = 2 * 128 * elt + (8 if b.scale_mode == 2 else 0)
    kv = int(np.asarray(ctx, dtype=np.int64).sum()) * kv_tok
    qo = N * hq * 128 * 2 * 2
    small = N * ld_s * 4 * 2 + N * 8 * topk * 4 + N * 4 + N * topk * 4 + b.num_reqs * 4 * 6 + N * 8
    return {"step": idx_k + N * 256 + kv + qo + small, "score": score_launch, "attn": kv + qo + N * 8 * topk * 4}


def cpu_baseline(b, rows):
    """The oracle as it stands, single-threaded, on `rows` of the workload."""
    from threadpoolctl import threadpool_limits

    from oracle import msa_oracle as O
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O.decode_step(b, rows=rows)
        dt = time.perf_counter() - t0
    return {"value": len(rows) / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(rows)} of {b.num_rows} rows of the {b.name} workload, full step "
                      f"(metadata, scores, pooling, selection, table, attention) in {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the decode path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_paged_msa_amd as msa
    import msa_synth as syn

    torch.cuda.set_device(0)
    msa.load()
    b = syn.config(args.workload)
    N, R, P, hq, topk, ld_s = b.num_rows, b.num_reqs, b.num_pages, b.num_q_heads, b.topk, b.ld_s
    per_copy = b.index_k.nbytes + b.k_cache.nbytes + b.v_cache.nbytes
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
    wsb = msa.msa_workspace_bytes(N, hq, 128 * topk, 0)
    ws = torch.empty((wsb,), dtype=torch.uint8, device=dev)

    def step(c):
        msa.msa_sparse_decode(batches[c], index_q, index_k, q, hq, kv, topk, b.sm_scale, out, table, ctx,
                              None, scores, ld_s, ws, wsb)

    for c in range(copies):
        step(c)
    torch.cuda.synchronize()
    ctx_host = ctx.cpu().numpy()
    nbytes = algorithmic_bytes(b, ctx_host)

    run = step
    if not args.eager:
        graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    step(c)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()

        def run(c):
            graphs[c].replay()

    for i in range(args.warmup):
        run(i % copies)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(i % copies)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec = (t1 - t0) / args.steps
    print(f"[bench] {args.workload}: {sec * 1e6:.2f} us/step over {args.steps} steps, {copies} copies",
          file=sys.stderr, flush=True)

    # per-entry-point times with events on the launching stream (eager launches)
    stream = torch.cuda.current_stream()

    def time_calls(fn, reps):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            evs[i][0].record(stream)
            fn(i % copies)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(e) for a, e in evs) / reps * 1e3   # us

    reps = max(args.steps, 20)
    t_meta = time_calls(lambda c: msa.msa_build_metadata(batches[c]), reps)
    t_score = time_calls(lambda c: msa.msa_index_score(batches[c], index_q, index_k, scores, ld_s), reps)
    t_topk = time_calls(lambda c: msa.msa_topk_block_table(batches[c], scores, ld_s, topk, table, ctx, None), reps)
    t_attn = time_calls(lambda c: msa.msa_sparse_paged_attn(q, N, hq, kv, table, 8 * topk, ctx, 128 * topk,
                                                            b.sm_scale, out, ws, wsb), reps)

    score_gbps = nbytes["score"] / (t_score * 1e-6) / 1e9
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
            if tj.get("workload") == args.workload and tj.get("kernel_source_hash") == source_hash():
                traffic = tj.get("score_bytes_per_launch")
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
        "config": {"workload": WORKLOAD_DESC[args.workload], "requests": R, "rows": N, "top_k": topk,
                   "q_heads": hq, "kv_heads": 1, "head_dim": 128, "seq_lens_sum": int(b.seq_lens.sum()),
                   "cache_copies_cycled": copies, "graphs": not args.eager},
        "step_hbm_gbps": nbytes["step"] / sec / 1e9,
        "step_hbm_frac": nbytes["step"] / sec / 1e9 / PEAK_HBM_GBPS,
        "step_algorithmic_bytes": nbytes["step"],
        "kernel_us": {"metadata": t_meta, "index_score": t_score, "topk_table": t_topk, "attention": t_attn},
        "roofline": {"kernel": "msa_score_kernel (msa_index_score)", "bound": "hbm", "achieved": score_gbps,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": score_gbps / PEAK_HBM_GBPS,
                     "traffic": traffic, "algorithmic_bytes": nbytes["score"], "avg_launch_us": t_score},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(b, list(range(min(N, 8))))
    print(json.dumps(res), flush=True)


def source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("msa_score.hip", "msa_internal.h"):
        with open(os.path.join(ROOT, "block_sparse_paged_msa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()

"""Throughput of the fused block-sparse paged decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--index bf16|fp8]

One step = metadata -> index score + pooling -> top-k + page-16 table + ctx ->
sparse paged attention + split merge (msa_sparse_decode) over one batch of the
named synthetic workload (default: the fp8 K/V decode batch, 11 requests x 1
row, L ~ U{32768..131072}, e4m3fn K/V with per-token-head scales, top-k 64,
16 query heads; --index fp8 stores the index keys as e4m3fn codes with
per-token scales). The step's inputs live in HBM; enough copies of the caches
at different addresses are cycled that at least 768 MB (three times the
256 MB Infinity Cache) stream through between two uses of one copy, in the
step loop and in the dominant-kernel loop alike. Steps are replayed from a
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
    p.add_argument("--workload", default="fp8_kv", choices=sorted(WORKLOAD_DESC))
    p.add_argument("--index", default="bf16", choices=("bf16", "fp8"),
                   help="index cache: bf16 keys, or e4m3fn codes with one fp32 scale per token")
    p.add_argument("--copies", type=int, default=0,
                   help="cache copies cycled (0: enough that >= 768 MB stream between two uses of a copy)")
    p.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying graphs")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="skip the other workloads' reduced lines")
    p.add_argument("--sweep", action="store_true",
                   help="instead of the bench line: the fused step on 16 fp8 K/V decode requests of 2K..64K "
                        "tokens each, one JSON line per length")
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


def time_insert(msa, torch, tokens=8192, copies=32, reps=32, decode=False):
    """msa_cache_insert of a prefill chunk (two sequences of 4096 new tokens, the
    mixed workload's prefill shape) into fp8 e4m3fn caches with per-token-head
    scales, index-K included: per-launch time over back-to-back launches in one
    graph, cycling `copies` sets of inputs and caches (>= 256 MB in all, so no
    launch finds its data in the Infinity Cache). Algorithmic bytes per token:
    K, V and index-K rows read (3 x 256 B) + the slot (4 B); fp8 K and V (2 x 128
    B), their scales (2 x 4 B) and the index-K row (256 B) written. With
    decode=True: one new token per request at a random slot of its own page
    (a decode step's insert), the same caches."""
    dev = "cuda"
    pages = max(tokens // 128, 64)
    g = torch.Generator(device="cpu").manual_seed(11)
    sets = []
    for c in range(copies):
        k_new = (torch.randn((tokens, 1, 128), generator=g) * 2).to(torch.bfloat16).to(dev)
        v_new = (torch.randn((tokens, 1, 128), generator=g) * 2).to(torch.bfloat16).to(dev)
        i_new = torch.randn((tokens, 128), generator=g).to(torch.bfloat16).to(dev)
        perm = torch.randperm(pages, generator=g)
        t = torch.arange(tokens)
        if decode:
            slots = (perm[:tokens] * 128 + torch.randint(0, 128, (tokens,), generator=g)).to(torch.int32).to(dev)
        else:
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


EXTRA_WORKLOADS = ("bf16_batch", "spec_decode", "mixed_prefill")   # timed too, as extra keys
CLEAN_BYTES = 768e6     # bytes streamed between two uses of one cache copy (3 x the 256 MB Infinity Cache)
MAX_COPIES = 64


def copies_for(b, idx_fp8):
    """Cache copies to cycle: the dominant kernel (the index score) touches
    every visible index key once, sum_r L_r x (256 B or 132 B), and a whole
    step touches more, so 1 + ceil(768 MB / that) copies keep at least 768 MB
    streaming between two uses of one copy in both loops (capped at 64 for
    the tiny workload, whose 0.5 MB step is latency-bound anyway)."""
    score_bytes = int(b.seq_lens.astype("int64").sum()) * (132 if idx_fp8 else 256)
    return min(MAX_COPIES, max(2, 1 + math.ceil(CLEAN_BYTES / max(score_bytes, 1))))


class Setup:
    """One workload on the device: `copies` replicas of its caches (each copy
    on its own pages), one batch struct per copy, the outputs, a workspace
    from msa_decode_workspace_bytes (the block-major path for prefill-sized
    launches) and the step / score launches of copy c."""

    def __init__(self, b, copies, idx_fp8, msa, torch, syn):
        import numpy as np
        self.b, self.copies, self.idx_fp8, self.msa, self.torch = b, copies, idx_fp8, msa, torch
        dev = "cuda"
        N, R, P, hq, topk, ld_s = b.num_rows, b.num_reqs, b.num_pages, b.num_q_heads, b.topk, b.ld_s

        def t16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()) if a.dtype == np.uint16 \
                else torch.from_numpy(np.ascontiguousarray(a).copy())

        def pool(a):
            one = t16(a).to(dev)
            out = torch.empty((copies,) + tuple(one.shape), dtype=one.dtype, device=dev)
            out[:] = one
            return out.view((copies * one.shape[0],) + tuple(one.shape[1:]))

        self.index_k = pool(b.index_k)
        self.index_scale = pool(b.index_scale) if idx_fp8 else None
        self.k_cache, self.v_cache = pool(b.k_cache), pool(b.v_cache)
        k_scale = v_scale = None
        if b.scale_mode == syn.SCALE_PER_TOKEN_HEAD:
            k_scale, v_scale = pool(b.k_scale), pool(b.v_scale)
        elif b.scale_mode == syn.SCALE_SCALAR:
            k_scale, v_scale = t16(b.k_scale).to(dev), t16(b.v_scale).to(dev)
        self.scales = (k_scale, v_scale)
        self.index_q, self.q = t16(b.index_q).to(dev), t16(b.q).to(dev)
        self.seq_lens = torch.from_numpy(b.seq_lens).to(dev)
        self.query_lens = torch.from_numpy(b.query_lens).to(dev)
        self.kv = msa.make_kv(self.k_cache, self.v_cache, b.kv_dtype, b.scale_mode, copies * P, k_scale, v_scale)
        i32 = dict(dtype=torch.int32, device=dev)
        self.batches, self.keep = [], []
        for c in range(copies):
            bt = torch.from_numpy(b.block_table + c * P).to(dev)
            meta = [torch.empty(R + 1, **i32) for _ in range(4)] + [torch.empty(N, **i32) for _ in range(2)]
            self.keep += [bt] + meta
            self.batches.append(msa.make_batch(self.seq_lens, self.query_lens, bt, *meta, R, N, b.max_seq_len,
                                               copies * P))
        self.out = torch.empty((N, hq, 128), dtype=torch.int16, device=dev)
        self.table = torch.empty((N, 8 * topk), **i32)
        self.ctx = torch.empty((N,), **i32)
        self.scores = torch.empty((N, ld_s), dtype=torch.float32, device=dev)
        self.wsb = msa.msa_decode_workspace_bytes(N, b.max_seq_len, hq, topk, 0)
        self.ws = torch.empty((self.wsb,), dtype=torch.uint8, device=dev)

    def step(self, c, sinks=None, lse=None):
        b, m = self.b, self.msa
        if self.idx_fp8 or sinks is not None or lse is not None:
            m.msa_sparse_decode_ex(self.batches[c], self.index_q, self.index_k, self.index_scale, self.q,
                                   b.num_q_heads, self.kv, b.topk, b.sm_scale, sinks, self.out, lse, self.table,
                                   self.ctx, None, self.scores, b.ld_s, self.ws, self.wsb)
        else:
            m.msa_sparse_decode(self.batches[c], self.index_q, self.index_k, self.q, b.num_q_heads, self.kv,
                                b.topk, b.sm_scale, self.out, self.table, self.ctx, None, self.scores, b.ld_s,
                                self.ws, self.wsb)

    def score(self, c):
        self.msa.msa_index_score_ex(self.batches[c], self.index_q, self.index_k, self.index_scale, self.scores,
                                    self.b.ld_s)


def graph_of(torch, fns):
    """One HIP graph holding the launches fns() in order (captured on a side
    stream, after one eager pass of each)."""
    stream = torch.cuda.current_stream()
    gs = torch.cuda.Stream()
    gs.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gs):
        for f in fns:
            f()
        with torch.cuda.graph(g, stream=gs):
            for f in fns:
                f()
    stream.wait_stream(gs)
    torch.cuda.synchronize()
    return g


def replay_us(torch, g, launches, runs=5, reps=1):
    """Median over `runs` of the time per launch of `reps` replays of g (which
    holds `launches` launches), HIP events on the replaying stream."""
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = []
    for _ in range(runs):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / (reps * launches))
    return sorted(out)[len(out) // 2]


def score_kernel_us(torch, st, reps=32):
    """The dominant kernel alone: `reps` back-to-back msa_index_score launches
    cycling the cache copies, captured in one graph and bracketed by HIP events
    on the launching stream."""
    g = graph_of(torch, [lambda i=i: st.score(i % st.copies) for i in range(reps)])
    return replay_us(torch, g, reps)


def step_figures(b, st, sec, t_score, ctx_host, table_host):
    """Throughput and rooflines of a timed step. Step bytes count each
    request's attended K/V once (rows of one request that keep the same
    blocks share them): the step's minimum HBM traffic."""
    import numpy as np
    nbytes = algorithmic_bytes(b, ctx_host)
    kv_unique = unique_kv_bytes(b, table_host, ctx_host)
    step_bytes = nbytes["step"] - nbytes["kv"] + kv_unique
    prefill = bool((b.query_lens > 64).any())
    step_gbps = step_bytes / sec / 1e9
    score_gbps = nbytes["score"] / (t_score * 1e-6) / 1e9
    res = {
        "rows_per_s": b.num_rows / sec, "us_per_step": sec * 1e6,
        "step_roofline": {"bound": "mfma" if prefill else "hbm", "achieved": step_gbps, "peak": PEAK_HBM_GBPS,
                          "unit": "GB/s", "frac": step_gbps / PEAK_HBM_GBPS, "algorithmic_bytes": step_bytes,
                          "us_per_step": sec * 1e6},
        "score_kernel": {"kernel": "msa_score_kernel (msa_index_score)", "bound": "hbm", "achieved": score_gbps,
                         "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": score_gbps / PEAK_HBM_GBPS,
                         "algorithmic_bytes": nbytes["score"], "avg_launch_us": t_score},
        "nbytes": nbytes,
    }
    if prefill:
        res["step_roofline"]["note"] = ("prefill rows: bound by the attention's MFMA work and its block partials; "
                                        "the HBM figure counts each request's attended K/V once")
        # requests of more than 64 rows are scored by the MFMA tile kernel:
        # 2 * 128 flops per (row, visible token) over every row of the launch
        pos = b.seq_lens.astype(np.int64) - b.query_lens.astype(np.int64)
        vis = sum(int(ql) * int(p0) + int(ql) * (int(ql) + 1) // 2 for p0, ql in zip(pos, b.query_lens))
        tflops = 2 * 128 * vis / (t_score * 1e-6) / 1e12
        res["score_mfma"] = {"kernels": "msa_score_kernel + msa_score_tile_kernel (one msa_index_score call)",
                             "bound": "mfma", "algorithmic_flop": 2 * 128 * vis, "us_per_call": t_score,
                             "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                             "frac": tflops / PEAK_BF16_TFLOPS}
    return res


def measure_extra(name, idx_fp8, steps, msa, torch, syn):
    """A reduced line for another workload: step time (graph replay over
    cache-clean copies), the score kernel alone, and both rooflines."""
    b = syn.config(name, index_dtype=syn.INDEX_FP8 if idx_fp8 else syn.INDEX_BF16)
    f = measure_batch(b, idx_fp8, steps, msa, torch, syn)
    f["workload"] = WORKLOAD_DESC[name]
    return f


def measure_batch(b, idx_fp8, steps, msa, torch, syn):
    """Step time (graph replay over cache-clean copies), the score kernel
    alone and both rooflines of one batch."""
    copies = copies_for(b, idx_fp8)
    st = Setup(b, copies, idx_fp8, msa, torch, syn)
    g = graph_of(torch, [lambda c=c: st.step(c) for c in range(copies)])
    reps = max(1, steps // copies)
    sec = replay_us(torch, g, copies, reps=reps) * 1e-6
    t_score = score_kernel_us(torch, st)
    f = step_figures(b, st, sec, t_score, st.ctx.cpu().numpy(), st.table.cpu().numpy())
    f.pop("nbytes")
    f.update({"rows": b.num_rows, "cache_copies_cycled": copies, "steps_timed": reps * copies})
    del st, g
    torch.cuda.empty_cache()
    return f


SWEEP_LENS = (2048, 4096, 8192, 16384, 32768, 65536)


def run_sweep(steps, msa, torch, syn):
    """--sweep: the fused step on 16 decode requests of one length each (fp8
    e4m3fn K/V with per-token-head scales, bf16 index, top-k 64, 16 query
    heads), for lengths of 2K to 64K tokens, one JSON line each: the step's
    algorithmic bytes grow with the length while the chain after the index
    scorer stays fixed, so the fraction of peak shows from what size a step is
    bound by HBM."""
    for i, L in enumerate(SWEEP_LENS):
        print(f"[bench] sweep: 16 requests of {L} tokens ...", file=sys.stderr, flush=True)
        b = syn.make_batch("sweep", 990 + i, [L] * 16, [1] * 16, topk=64, num_q_heads=16, kv_dtype=syn.KV_FP8,
                           scale_mode=syn.SCALE_PER_TOKEN_HEAD)
        f = measure_batch(b, False, steps, msa, torch, syn)
        print(json.dumps({"sweep": "fp8 K/V decode, 16 requests x 1 row, top-k 64, 16 q heads", "seq_len": L,
                          "us_per_step": f["us_per_step"],
                          "step_algorithmic_mb": f["step_roofline"]["algorithmic_bytes"] / 1e6,
                          "step_frac": f["step_roofline"]["frac"], "score_us": f["score_kernel"]["avg_launch_us"],
                          "score_frac": f["score_kernel"]["frac"], "cache_copies_cycled": f["cache_copies_cycled"]}),
              flush=True)


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

    if args.sweep:
        torch.cuda.set_device(0)
        msa.load()
        run_sweep(args.steps, msa, torch, syn)
        return

    idx_fp8 = args.index == "fp8"
    b = syn.config(args.workload, index_dtype=syn.INDEX_FP8 if idx_fp8 else syn.INDEX_BF16)
    cpu_par = None
    if not args.no_cpu_baseline:  # before the GPU is touched (the pool forks this process)
        print("[bench] cpu baseline, all cores (oracle) ...", file=sys.stderr, flush=True)
        cpu_par = cpu_baseline_parallel(b, list(range(min(b.num_rows, 8))))
    torch.cuda.set_device(0)
    msa.load()
    copies = args.copies or copies_for(b, idx_fp8)
    st = Setup(b, copies, idx_fp8, msa, torch, syn)
    N, hq = b.num_rows, b.num_q_heads

    for c in range(copies):
        st.step(c)
    torch.cuda.synchronize()
    if args.counters:
        # counter pass: plain copies of known size, then the dominant kernel
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(8):
            torch.mul(src, 1, out=dst)   # an elementwise kernel: reads and writes COPY_BYTES
        torch.cuda.synchronize()
        for i in range(8):
            st.score(i % copies)
        torch.cuda.synchronize()
        print(json.dumps({"counters_pass": args.workload, "copy_bytes": COPY_BYTES,
                          "score_algorithmic_bytes": algorithmic_bytes(b, st.ctx.cpu().numpy())["score"]}))
        return
    ctx_host, table_host = st.ctx.cpu().numpy(), st.table.cpu().numpy()

    if args.eager:
        def run_steps(k):
            for i in range(k):
                st.step(i % copies)
        graphs = None
    else:
        # the timed steps are one graph of exactly `steps` steps (cycling the
        # cache copies), so that the host launches them with one replay; the
        # warm-up steps are another graph, and one graph per copy serves the
        # single-step latency samples below
        g_warm = graph_of(torch, [lambda i=i: st.step(i % copies) for i in range(max(args.warmup, 1))])
        g_timed = graph_of(torch, [lambda i=i: st.step(i % copies) for i in range(args.steps)])
        graphs = [graph_of(torch, [lambda c=c: st.step(c)]) for c in range(copies)]

        def run_steps(k):
            (g_timed if k == args.steps else g_warm).replay()

    if args.warmup > 0 or args.eager:
        run_steps(args.warmup)
    # the K timed steps, bracketed by synchronisations and timed with the
    # host's wall clock (graph launch and final wait included); HIP events on
    # the launching stream give the GPU's own time for the same steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    run_steps(args.steps)
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec = (t1 - t0) / args.steps
    sec_events = ev0.elapsed_time(ev1) * 1e-3 / args.steps
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
        if graphs is None:
            st.step(c)
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

    t_score = score_kernel_us(torch, st)
    fig = step_figures(b, st, sec, t_score, ctx_host, table_host)
    traffic = None
    tpath = os.path.join(ROOT, "profiles", TRAFFIC_FILE.format(tag(args.workload, args.index)))
    if os.path.exists(tpath):
        try:
            tj = json.load(open(tpath))
            if tj.get("kernel_source_hash") == source_hash():
                traffic = tj.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    roof = dict(fig["score_kernel"])
    roof["traffic"] = traffic

    res = {
        "metric": METRIC,
        "value": N / sec,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "ms_per_step_gpu_events": sec_events * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if b.kv_dtype == 0 else "fp8-kv/bf16",
        "data": "synthetic (seeded splitmix64 N(0,1) values, random page permutation)",
        "config": {"workload": WORKLOAD_DESC[args.workload] + (
                       ", fp8 e4m3fn index keys + per-token scales" if idx_fp8 else ""),
                   "requests": b.num_reqs, "rows": N, "top_k": b.topk,
                   "q_heads": hq, "kv_heads": 1, "head_dim": 128, "seq_lens_sum": int(b.seq_lens.sum()),
                   "cache_copies_cycled": copies, "bytes_between_copy_reuses_min": (copies - 1) *
                   fig["score_kernel"]["algorithmic_bytes"], "graphs": not args.eager},
        "step_roofline": fig["step_roofline"],
        "roofline": roof,
        "step_latency": step_lat,
    }
    if "score_mfma" in fig:
        res["score_mfma"] = fig["score_mfma"]
    res["cache_insert"] = time_insert(msa, torch)
    dec = time_insert(msa, torch, tokens=11, decode=True)
    res["cache_insert"]["decode_step"] = {"tokens": 11, "slots": "one per request, scattered",
                                          "us_per_launch": dec["us_per_launch"]}

    # the same step through msa_sparse_decode_ex: LSE written, per-head sinks
    # applied; both variants timed here the same way (one graph of `copies`
    # steps, replayed)
    sinks = torch.linspace(-1.0, 2.0, hq, device="cuda", dtype=torch.float32)
    lse = torch.empty((N, hq), dtype=torch.float32, device="cuda")
    reps_g = max(1, 192 // copies)
    g_lse = graph_of(torch, [lambda c=c: st.step(c, sinks, lse) for c in range(copies)])
    g_plain = graph_of(torch, [lambda c=c: st.step(c) for c in range(copies)])
    res["lse_sinks"] = {"entry": "msa_sparse_decode_ex", "us_per_step": replay_us(torch, g_lse, copies, reps=reps_g),
                        "plain_us_per_step": replay_us(torch, g_plain, copies, reps=reps_g), "rows": N,
                        "q_heads": hq}
    del st, g_lse, g_plain, graphs
    if not args.eager:
        del g_warm, g_timed
    torch.cuda.empty_cache()
    if args.workload == "fp8_kv" and not idx_fp8 and not args.no_extras:
        res["other_workloads"] = {}
        for name in EXTRA_WORKLOADS:
            print(f"[bench] extra workload {name} ...", file=sys.stderr, flush=True)
            res["other_workloads"][name] = measure_extra(name, False, 200, msa, torch, syn)
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
             "python3 -u bench.py --workload {workload}{index} --steps 50 --warmup 10 --no-cpu-baseline --no-extras")


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
            "--no-cpu-baseline --no-extras")
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

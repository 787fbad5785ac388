"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.

Bars: bit-exact metadata, selections, sparse tables and context lengths (the
selection is checked on the device's own fp32 block scores); block scores
within 1e-3 * max(|oracle|, 1) with exact -inf past each row's block count;
attention within 2e-2 absolute (bf16 K/V) or 6e-2 (fp8 K/V) of the oracle run
on the device's own table and context lengths, and elementwise within the
tighter detector bar of tests/bars.py (5e-4 + 2^-8 (|oracle| + weighted mean
|V|)), which a missing or doubled block cannot meet.
"""
import dataclasses
import functools
import math

import numpy as np
import pytest
import torch

import block_sparse_paged_msa_amd as msa
import msa_synth as syn
from oracle import msa_oracle as O
from tests import bars
from tests import helpers as H

pytestmark = pytest.mark.gpu

SCORE_RTOL = 1e-3
ATOL_BF16 = bars.ATOL_BF16
ATOL_FP8 = bars.ATOL_FP8


def atol_for(b):
    return bars.contract_atol(b.kv_dtype)


def check_scores(b, gpu, rows):
    ref = O.block_scores(b.index_q, b.index_k, b.block_table, b.seq_lens, b.query_lens, b.ld_s, rows=rows,
                         index_scale=b.index_scale)
    meta = O.build_metadata(b.seq_lens, b.query_lens)
    for n in rows:
        nb = O.num_blocks(O.visible_keys(meta["row_pos"][n]))
        g, o = gpu[n], ref[n]
        assert np.all(np.isneginf(g[nb:])), f"row {n}: tail past nb={nb} is not -inf"
        err = np.abs(g[:nb] - o[:nb]) / np.maximum(np.abs(o[:nb]), 1.0)
        assert np.all(np.isfinite(g[:nb])), f"row {n}: non-finite score"
        assert err.max(initial=0.0) <= SCORE_RTOL, f"row {n}: score rel err {err.max()}"
    return ref


def check_selection(b, gpu_scores, table, ctx, sel, rows):
    """Bit-exact against the oracle selector fed the device's fp32 scores."""
    meta = O.build_metadata(b.seq_lens, b.query_lens)
    for n in rows:
        r = int(meta["row_req"][n])
        v = O.visible_keys(meta["row_pos"][n])
        nb = O.num_blocks(v)
        s = O.select_blocks(gpu_scores[n].astype(np.float64), nb, b.topk)
        assert sel[n].tolist() == O.selection_row_outputs(s, b.topk).tolist(), f"row {n}: selection"
        assert table[n].tolist() == O.sparse_table_row(s, b.block_table[r], b.topk).tolist(), f"row {n}: table"
        assert ctx[n] == O.context_length(s, v), f"row {n}: ctx"


def check_selection_valid(b, oracle_scores, sel, rows):
    """The device's choice is a valid top-k of the oracle's own scores within
    the score tolerance (near-ties may fall either way)."""
    meta = O.build_metadata(b.seq_lens, b.query_lens)
    for n in rows:
        nb = O.num_blocks(O.visible_keys(meta["row_pos"][n]))
        kk = min(b.topk, nb)
        chosen = [int(x) for x in sel[n][:kk]]
        s = oracle_scores[n][:nb]
        tol = SCORE_RTOL * np.maximum(np.abs(s), 1.0) * 2
        thr = np.sort(s)[::-1][kk - 1]
        others = np.setdiff1d(np.arange(nb), chosen)
        assert np.all(s[chosen] + tol[chosen] >= thr), f"row {n}: a kept block is clearly below the k-th score"
        if len(others):
            assert np.all(s[others] - tol[others] <= thr), f"row {n}: a dropped block is clearly above the k-th"


def check_metadata(b, got):
    """Bit-exact batch metadata, including the per-request unit counts."""
    ref = O.build_metadata(b.seq_lens, b.query_lens)
    for key in ("cu_seqlens_q", "cu_seqlens_k", "cu_blocks", "row_req", "row_pos"):
        assert got[key].tolist() == ref[key].tolist(), key
    L, ql = b.seq_lens.astype(np.int64), b.query_lens.astype(np.int64)
    units = [0] + np.cumsum(-(-L // 128) * -(-ql // 64)).tolist()
    assert got["cu_units"].tolist() == units, "cu_units"


def check_attention(b, out, table, ctx, rows):
    """Contract bar on the max abs error, then the detector bar elementwise."""
    ref, amean = bars.oracle_and_abs_mean(b, table, ctx, rows)
    err = np.abs(out[rows] - ref)
    assert err.max() <= atol_for(b), f"attention max abs err {err.max()} (rows {rows})"
    ex = bars.detect_excess(out[rows], ref, amean)
    assert ex <= 0, f"attention outside the detector bar by {ex} (max abs err {err.max()}, rows {rows})"
    return err.max()


# ---------------------------------------------------------------------------
# metadata
# ---------------------------------------------------------------------------
META_CASES = [
    ([5, 300, 128, 0, 4097], [1, 4, 2, 0, 1]),
    ([1], [1]),
    ([16384] * 6 + [32768] * 2, [1] * 6 + [4096] * 2),
    ([0, 0, 7, 0], [0, 0, 7, 0]),
]


@pytest.mark.parametrize("case", range(len(META_CASES) + 3))
def test_metadata_bitexact(gpu_lib, case):
    if case < len(META_CASES):
        L, ql = META_CASES[case]
        b = syn.make_batch("meta", case, L, ql, topk=2, num_q_heads=16, max_seq_len=max(max(L), 1))
    else:
        b = syn.random_batch(40 + case, num_reqs=37 + 500 * (case - len(META_CASES)), max_len=3000, max_q=9)
    d = H.upload(b)
    check_metadata(b, H.run_metadata(d))


# ---------------------------------------------------------------------------
# index scores
# ---------------------------------------------------------------------------
SCORE_CASES = [
    dict(L=[2048], ql=[1]),
    dict(L=[300, 129, 1, 700, 128], ql=[1, 3, 1, 4, 2]),
    dict(L=[1000, 5000], ql=[70, 33]),                 # several 16-row tiles and row groups
    dict(L=[4000, 0, 257], ql=[130, 0, 17], max_seq_len=8192),  # empty request, wide ld_s
]


@pytest.mark.parametrize("case", range(len(SCORE_CASES)))
def test_index_scores(gpu_lib, case):
    c = SCORE_CASES[case]
    b = syn.make_batch("score", 60 + case, c["L"], c["ql"], topk=4, num_q_heads=16,
                       max_seq_len=c.get("max_seq_len"))
    d = H.upload(b)
    H.run_metadata(d)
    gpu = H.run_scores(d)
    check_scores(b, gpu, list(range(b.num_rows)))


def test_index_scores_closed_form(gpu_lib):
    # all-ones keys and query: every visible token scores exactly 128
    b = syn.make_batch("ones", 70, [700, 64], [3, 1], topk=2, num_q_heads=16)
    one = np.uint16(0x3F80)
    b.index_k[:] = one
    b.index_q[:] = one
    d = H.upload(b)
    H.run_metadata(d)
    gpu = H.run_scores(d)
    assert np.all(gpu[:, :1] == 128.0)
    assert gpu[0, :6].tolist() == [128.0] * 6 and np.isneginf(gpu[0, 6:]).all()


# ---------------------------------------------------------------------------
# top-k, page-16 table, context length
# ---------------------------------------------------------------------------
def _crafted_scores(b, mode, seed):
    rng = syn.SplitMix64(seed)
    s = rng.normal(b.num_rows * b.ld_s).reshape(b.num_rows, b.ld_s)
    if mode == "ties":
        s = np.round(s * 2) / 2
    elif mode == "zeros":
        s = np.where(rng.uniform(s.size).reshape(s.shape) < 0.5, 0.0, -0.0)
    elif mode == "equal":
        s = np.full_like(s, 3.25)
    elif mode == "few_distinct":
        s = np.floor(rng.uniform(s.size).reshape(s.shape) * 3) - 1.0
    return s.astype(np.float32)


@functools.lru_cache(maxsize=1)
def _topk_batch():
    L = [128000, 5000, 129, 1, 2047, 640, 0, 77]
    ql = [1, 2, 1, 1, 4, 3, 0, 77]
    return syn.make_batch("topk", 80, L, ql, topk=1, num_q_heads=16, max_seq_len=131072, data=False)


@functools.lru_cache(maxsize=1)
def _topk_batch_long():
    # rows of more than 1024 blocks: the keys past the 1024 a wave holds in
    # registers are read again from memory, chunk by chunk
    L = [140000, 131073, 5000, 1]
    ql = [1, 2, 1, 1]
    return syn.make_batch("topk_long", 85, L, ql, topk=1, num_q_heads=16, max_seq_len=140032, data=False)


@pytest.mark.parametrize("mode", ["normal", "ties", "zeros", "equal", "few_distinct"])
@pytest.mark.parametrize("topk", [1, 3, 16, 64, 1500])
def test_topk_bitexact(gpu_lib, mode, topk):
    b = dataclasses.replace(_topk_batch(), topk=topk)
    d = H.upload(b)
    H.run_metadata(d)
    s = _crafted_scores(b, mode, 81 + topk)
    table, ctx, sel = H.run_topk(d, s)
    check_selection(b, s, table, ctx, sel, range(b.num_rows))


@pytest.mark.parametrize("mode", ["normal", "ties", "few_distinct"])
@pytest.mark.parametrize("topk", [1, 64, 1500])
def test_topk_bitexact_long_rows(gpu_lib, mode, topk):
    b = dataclasses.replace(_topk_batch_long(), topk=topk)
    assert b.ld_s > 1024
    d = H.upload(b)
    H.run_metadata(d)
    s = _crafted_scores(b, mode, 86 + topk)
    table, ctx, sel = H.run_topk(d, s)
    check_selection(b, s, table, ctx, sel, range(b.num_rows))


# ---------------------------------------------------------------------------
# attention on a given table
# ---------------------------------------------------------------------------
ATTN_CASES = [
    dict(kv=syn.KV_BF16, sm=syn.SCALE_NONE, hq=16),
    dict(kv=syn.KV_BF16, sm=syn.SCALE_NONE, hq=8),
    dict(kv=syn.KV_BF16, sm=syn.SCALE_NONE, hq=24),
    dict(kv=syn.KV_FP8, sm=syn.SCALE_SCALAR, hq=16),
    dict(kv=syn.KV_FP8, sm=syn.SCALE_PER_TOKEN_HEAD, hq=16),
    dict(kv=syn.KV_BF16, sm=syn.SCALE_PER_TOKEN_HEAD, hq=16),
]


@pytest.mark.parametrize("case", range(len(ATTN_CASES)))
def test_attention_on_device_table(gpu_lib, case):
    c = ATTN_CASES[case]
    L = [9000, 700, 129, 1, 20000, 3000]
    ql = [1, 2, 1, 1, 1, 3]
    b = syn.make_batch("attn", 90 + case, L, ql, topk=24, num_q_heads=c["hq"], kv_dtype=c["kv"],
                       scale_mode=c["sm"])
    d = H.upload(b)
    H.run_metadata(d)
    scores = H.run_scores(d)
    table, ctx, sel = H.run_topk(d, scores)
    out = H.run_attn(d, table, ctx, max_ctx=128 * b.topk)
    check_attention(b, out, table, ctx, list(range(b.num_rows)))


def test_attention_zero_context_rows_give_zeros(gpu_lib):
    b = syn.make_batch("attn0", 99, [500, 300], [1, 1], topk=4, num_q_heads=16)
    d = H.upload(b)
    table = np.zeros((2, 32), np.int32)
    table[1, :8] = np.arange(8) + 8 * int(b.block_table[1, 0])
    ctx = np.array([0, 100], np.int32)
    out = H.run_attn(d, table, ctx, max_ctx=512)
    assert np.all(out[0] == 0.0)
    check_attention(b, out, table, ctx, [1])


# ---------------------------------------------------------------------------
# the fused decode step
# ---------------------------------------------------------------------------
FUSED_CASES = [
    ([9000, 700, 129, 1, 20000], [1, 2, 1, 1, 4]),
    ([9000, 0, 700, 129, 300, 1], [1, 0, 2, 0, 3, 1]),   # empty request, requests with no rows
]


@pytest.mark.parametrize("case", range(len(FUSED_CASES)))
def test_fused_decode_equals_steps_and_oracle(gpu_lib, case):
    L, ql = FUSED_CASES[case]
    b = syn.make_batch("fused", 110 + case, L, ql, topk=16, num_q_heads=16)
    d = H.upload(b)
    o = H.alloc_decode(d)
    H.run_decode(d, o)
    check_metadata(b, H.read_metadata(d))  # written by the fused step
    scores = o.scores.cpu().numpy()
    table, ctx, sel = o.table.cpu().numpy(), o.ctx.cpu().numpy(), o.sel.cpu().numpy()
    out = H.bf16_to_np(o.out)
    rows = list(range(b.num_rows))
    ref_scores = check_scores(b, scores, rows)
    check_selection(b, scores, table, ctx, sel, rows)
    check_selection_valid(b, ref_scores, sel, rows)
    check_attention(b, out, table, ctx, rows)
    # the standalone entry points give the same bits
    H.run_metadata(d)
    s2 = H.run_scores(d)
    assert np.array_equal(s2, scores)
    t2, c2, sel2 = H.run_topk(d, s2)
    assert np.array_equal(t2, table) and np.array_equal(c2, ctx) and np.array_equal(sel2, sel)
    out2 = H.run_attn(d, t2, c2, max_ctx=128 * b.topk)
    assert np.array_equal(out2, out)
    # scores kept in the workspace instead of a caller buffer: same outputs
    o3 = H.alloc_decode(d, with_scores=False)
    H.run_decode(d, o3, with_scores=False)
    assert torch.equal(o3.out, o.out) and torch.equal(o3.table, o.table)


FUSED_SHAPES = [
    # (name, lengths, query rows, top-k, query heads): many splits per row
    # (the merge takes several rounds), and head groups past the first
    ("topk300", [140000, 70000], [1, 2], 300, 16),
    ("hq24", [9000, 3000, 20000], [1, 3, 2], 24, 24),
    ("hq8", [5000, 129, 70000], [2, 1, 1], 40, 8),
    # the most query heads the library takes: eight head groups
    ("hq128", [6000, 20000], [1, 2], 16, 128),
]


@pytest.mark.parametrize("case", range(len(FUSED_SHAPES)))
def test_fused_decode_shapes(gpu_lib, case):
    name, L, ql, topk, hq = FUSED_SHAPES[case]
    b = syn.make_batch(name, 140 + case, L, ql, topk=topk, num_q_heads=hq)
    print(f"[fused] {name} rows={b.num_rows} topk={topk} hq={hq}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    H.run_decode(d, o)
    check_metadata(b, H.read_metadata(d))
    scores = o.scores.cpu().numpy()
    table, ctx, sel = o.table.cpu().numpy(), o.ctx.cpu().numpy(), o.sel.cpu().numpy()
    rows = list(range(b.num_rows))
    check_scores(b, scores, rows)
    check_selection(b, scores, table, ctx, sel, rows)
    check_attention(b, H.bf16_to_np(o.out), table, ctx, rows)


@pytest.mark.parametrize("sm_scale", [4.0, 1e-3])
def test_fused_decode_extreme_softmax_scale(gpu_lib, sm_scale):
    """A sharp softmax (sm_scale 4: logits of standard deviation ~45, nearly
    one token per head) and a flat one (sm_scale 1e-3: nearly equal weights)
    through the per-row path with many splits a row: the running max and the
    merge's rescaling keep both bars."""
    b = syn.make_batch("smscale", 870, [70000, 9000, 300], [1, 2, 1], topk=64, num_q_heads=16,
                       kv_dtype=syn.KV_FP8, scale_mode=syn.SCALE_PER_TOKEN_HEAD)
    b = dataclasses.replace(b, sm_scale=sm_scale)
    print(f"[fused] sm_scale={sm_scale} rows={b.num_rows}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    H.run_decode(d, o)
    table, ctx, sel = o.table.cpu().numpy(), o.ctx.cpu().numpy(), o.sel.cpu().numpy()
    rows = list(range(b.num_rows))
    check_selection(b, o.scores.cpu().numpy(), table, ctx, sel, rows)
    out = H.bf16_to_np(o.out)
    assert np.isfinite(out).all()
    check_attention(b, out, table, ctx, rows)


RANDOM_KV = [(syn.KV_BF16, syn.SCALE_NONE), (syn.KV_BF16, syn.SCALE_PER_TOKEN_HEAD),
             (syn.KV_FP8, syn.SCALE_SCALAR), (syn.KV_FP8, syn.SCALE_PER_TOKEN_HEAD)]


@pytest.mark.parametrize("seed", range(16))
def test_random_batches_match_oracle(gpu_lib, seed):
    """Small batches whose shape is drawn from the seed (1 to 12 requests,
    lengths 0 to 12000 so that empty requests and partial last blocks occur,
    0 to 4 query rows each, top-k, query heads, K/V dtype and scale mode,
    index dtype) through the fused step: metadata, selections, tables and
    context lengths bit-exact, scores and attention within their bars, on
    every row."""
    rng = syn.SplitMix64(7000 + seed)
    R = int(rng.integers(1, 12, 1)[0])
    L = rng.integers(0, 12000, R)
    L = np.where(rng.uniform(R) < 0.2, L // 128 * 128, L)   # whole blocks only
    L = np.where(rng.uniform(R) < 0.2, 0, L)                 # empty requests
    ql = np.minimum(rng.integers(0, 4, R), L)
    if ql.sum() == 0:
        L[0], ql[0] = max(int(L[0]), 1), 1
    pick = lambda opts: opts[int(rng.integers(0, len(opts) - 1, 1)[0])]
    topk, hq = pick([1, 2, 5, 16, 33, 64]), pick([8, 16, 24, 40, 64])
    kv, sm = pick(RANDOM_KV)
    idx = pick([syn.INDEX_BF16, syn.INDEX_FP8])
    b = syn.make_batch("random_step", 7000 + seed, L, ql, topk=topk, num_q_heads=hq, kv_dtype=kv, scale_mode=sm,
                       index_dtype=idx)
    print(f"[random] seed {seed}: L={L.tolist()} ql={ql.tolist()} topk={topk} hq={hq} kv={kv} scale={sm} "
          f"index={idx}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    H.run_decode(d, o)
    check_metadata(b, H.read_metadata(d))
    scores = o.scores.cpu().numpy()
    table, ctx, sel = o.table.cpu().numpy(), o.ctx.cpu().numpy(), o.sel.cpu().numpy()
    rows = list(range(b.num_rows))
    check_scores(b, scores, rows)
    check_selection(b, scores, table, ctx, sel, rows)
    out = H.bf16_to_np(o.out)
    assert np.isfinite(out).all()
    check_attention(b, out, table, ctx, rows)


TIE_SHAPES = [
    # (longest row, lengths): rows past 1024 blocks select wave by wave with
    # the last keys re-read from memory; rows of at most 1024 or 256 blocks
    # select with the four waves sharing one histogram
    (140032, [140000, 33000, 9000, 129, 1, 2047]),
    (131072, [131000, 33000, 9000, 129, 1, 2047]),
    (32768, [32768, 20000, 9000, 129, 1, 2047]),
]


@pytest.mark.parametrize("shape", range(len(TIE_SHAPES)))
@pytest.mark.parametrize("topk", [1, 5, 16, 64])
def test_fused_selection_with_tied_scores(gpu_lib, topk, shape):
    """Index queries and keys in {-1, 0, 1}: every token score is an integer,
    so many blocks share their pooled maximum and the cut falls inside a tie
    (the lowest block ids are kept)."""
    max_len, L = TIE_SHAPES[shape]
    ql = [1, 1, 2, 1, 1, 3]
    b = syn.make_batch("ties", 130 + topk + 7 * shape, L, ql, topk=topk, num_q_heads=16, max_seq_len=max_len)
    tern = lambda x: syn.to_bf16_bits(np.clip(np.round(O.bf16_to_f64(x)), -1.0, 1.0))
    b = dataclasses.replace(b, index_q=tern(b.index_q), index_k=tern(b.index_k))
    print(f"[ties] topk={topk} rows={b.num_rows} pages={b.num_pages}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    H.run_decode(d, o)
    scores = o.scores.cpu().numpy()
    table, ctx, sel = o.table.cpu().numpy(), o.ctx.cpu().numpy(), o.sel.cpu().numpy()
    rows = list(range(b.num_rows))
    ref = check_scores(b, scores, rows)
    meta = O.build_metadata(b.seq_lens, b.query_lens)
    straddled = 0
    for n in rows:
        nb = O.num_blocks(O.visible_keys(meta["row_pos"][n]))
        assert np.array_equal(scores[n][:nb], ref[n][:nb].astype(np.float32)), f"row {n}: integer scores differ"
        if topk < nb:
            srt = np.sort(ref[n][:nb])[::-1]
            straddled += int(srt[topk - 1] == srt[topk])
    assert straddled >= 1, "the crafted inputs should put the cut inside a tie"
    check_selection(b, scores, table, ctx, sel, rows)
    check_attention(b, H.bf16_to_np(o.out), table, ctx, rows)


PREFILL_CASES = [
    # prefill-shaped batches (>= 1024 rows): long requests around a one-row
    # request, fp8 with both scale modes, a row bound past 1024 blocks
    dict(L=[20000, 5000, 3000], ql=[600, 1, 500], kv=syn.KV_BF16, sm=syn.SCALE_NONE, topk=24),
    dict(L=[9000, 140000, 700], ql=[300, 720, 17], kv=syn.KV_FP8, sm=syn.SCALE_PER_TOKEN_HEAD, topk=40),
    dict(L=[4100, 2000], ql=[1000, 37], kv=syn.KV_FP8, sm=syn.SCALE_SCALAR, topk=8),
]


@pytest.mark.parametrize("case", range(len(PREFILL_CASES)))
def test_fused_prefill_batches(gpu_lib, case):
    c = PREFILL_CASES[case]
    b = syn.make_batch("prefill", 150 + case, c["L"], c["ql"], topk=c["topk"], num_q_heads=16,
                       kv_dtype=c["kv"], scale_mode=c["sm"])
    print(f"[prefill] case {case} rows={b.num_rows} ld_s={b.ld_s}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    H.run_decode(d, o)
    check_metadata(b, H.read_metadata(d))
    scores = o.scores.cpu().numpy()
    table, ctx, sel = o.table.cpu().numpy(), o.ctx.cpu().numpy(), o.sel.cpu().numpy()
    check_selection(b, scores, table, ctx, sel, range(b.num_rows))
    out = H.bf16_to_np(o.out)
    assert np.isfinite(out).all(), "every row's output is written"
    rows = _sample_rows(b, 16, 160 + case)
    check_scores(b, scores, rows)
    check_attention(b, out, table, ctx, rows)


def test_two_streams_at_once_match_one_at_a_time(gpu_lib):
    """Two fused steps enqueued on two streams with nothing ordering them
    (each with its own workspace and outputs; the per-row path and the
    block-major path side by side) give the bits each gives alone: no call
    depends on device state another call writes."""
    cases = [(syn.config("spec_decode"), False),
             (syn.make_batch("streams_bm", 890, [6000, 3000], [2100, 1], topk=8, num_q_heads=16), True)]
    devs, refs, outs = [], [], []
    for b, bm in cases:
        d = H.upload(b)
        devs.append(d)
        for dst in (refs, outs):
            o = H.alloc_decode(d)
            if bm:
                wsb = msa.msa_decode_workspace_bytes(b.num_rows, b.max_seq_len, b.num_q_heads, b.topk, 0)
                o.ws, o.wsb = torch.empty((wsb,), dtype=torch.uint8, device="cuda"), wsb
            dst.append(o)
    for d, o in zip(devs, refs):
        H.run_decode(d, o)
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    print("[streams] two steps on two streams, three rounds", flush=True)
    for _ in range(3):
        for d, o, st in zip(devs, outs, streams):
            with torch.cuda.stream(st):
                H.run_decode(d, o)
    torch.cuda.synchronize()
    for o, r in zip(outs, refs):
        for field in ("out", "table", "ctx", "sel", "scores"):
            assert torch.equal(getattr(o, field), getattr(r, field)), field


def test_fused_decode_repeat_and_graph_replay_bitwise(gpu_lib):
    b = syn.make_batch("graph", 120, [20000, 3000, 7000], [4, 1, 2], topk=16, num_q_heads=16)
    d = H.upload(b)
    o = H.alloc_decode(d)
    H.run_decode(d, o)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o.out, o.table, o.ctx, o.sel, o.scores)]
    H.run_decode(d, o)
    for t, r in zip((o.out, o.table, o.ctx, o.sel, o.scores), ref):
        assert torch.equal(t, r)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        H.run_decode(d, o)           # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        H.run_decode(d, o)
    for rep in range(3):
        o.out.zero_()
        o.table.fill_(-1)
        o.ws.fill_(0x3F3F3F3F)       # garbage counters: the step resets them in-stream
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip((o.out, o.table, o.ctx, o.sel, o.scores), ref):
            assert torch.equal(t, r), f"replay {rep}"


def _permute_pages(b, seed):
    P = b.num_pages
    pi = syn.SplitMix64(seed).permutation(P)
    nb = syn.Batch(**{f: getattr(b, f) for f in b.__dataclass_fields__})
    nb.block_table = np.where(b.block_table >= 0, pi[b.block_table], b.block_table).astype(np.int32)
    nb.index_k = np.empty_like(b.index_k)
    nb.index_k[pi] = b.index_k
    sub = (8 * pi[:, None] + np.arange(8)[None, :]).reshape(-1)
    nb.k_cache = np.empty_like(b.k_cache)
    nb.k_cache[sub] = b.k_cache
    nb.v_cache = np.empty_like(b.v_cache)
    nb.v_cache[sub] = b.v_cache
    if b.scale_mode == syn.SCALE_PER_TOKEN_HEAD:
        nb.k_scale = np.empty_like(b.k_scale)
        nb.k_scale[sub] = b.k_scale
        nb.v_scale = np.empty_like(b.v_scale)
        nb.v_scale[sub] = b.v_scale
    return nb


def test_physical_page_permutation_changes_no_output_bit(gpu_lib):
    b = syn.make_batch("perm", 130, [9000, 3000], [1, 3], topk=8, num_q_heads=16, kv_dtype=syn.KV_FP8,
                       scale_mode=syn.SCALE_PER_TOKEN_HEAD)
    outs = []
    for bb in (b, _permute_pages(b, 131)):
        d = H.upload(bb)
        o = H.alloc_decode(d)
        H.run_decode(d, o)
        outs.append((o.out.cpu(), o.ctx.cpu(), o.sel.cpu(), o.scores.cpu()))
    for x, y in zip(*outs):
        assert torch.equal(x, y)


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------
@functools.lru_cache(maxsize=1)
def _config(name, scale_mode, index_dtype=syn.INDEX_BF16):
    return syn.config(name, scale_mode=scale_mode, index_dtype=index_dtype)


def _sample_rows(b, k, seed):
    N = b.num_rows
    if N <= k:
        return list(range(N))
    meta = O.build_metadata(b.seq_lens, b.query_lens)
    rows = set()
    for r in range(b.num_reqs):                  # first and last row of each request
        lo, hi = int(meta["cu_seqlens_q"][r]), int(meta["cu_seqlens_q"][r + 1])
        if hi > lo:
            rows.update([lo, hi - 1])
    rng = syn.SplitMix64(seed)
    rows.update(int(x) for x in rng.integers(0, N - 1, k))
    return sorted(rows)


@pytest.mark.parametrize("name,scale_mode,index_dtype", [
    ("tiny", None, 0), ("bf16_batch", None, 0), ("spec_decode", None, 0),
    ("fp8_kv", syn.SCALE_PER_TOKEN_HEAD, 0), ("fp8_kv", syn.SCALE_SCALAR, 0), ("mixed_prefill", None, 0),
    # the same workloads on an fp8 index cache
    ("bf16_batch", None, syn.INDEX_FP8), ("fp8_kv", syn.SCALE_PER_TOKEN_HEAD, syn.INDEX_FP8),
    ("mixed_prefill", None, syn.INDEX_FP8),
])
def test_workload_parity(gpu_lib, name, scale_mode, index_dtype):
    _workload_parity(name, scale_mode, index_dtype, bench_workspace=False)


@pytest.mark.parametrize("name,index_dtype", [("mixed_prefill", 0), ("mixed_prefill", syn.INDEX_FP8),
                                              ("bf16_batch", 0), ("fp8_kv", 0)])
def test_workload_parity_bench_launch(gpu_lib, name, index_dtype):
    """The launch bench.py times: the workspace from msa_decode_workspace_bytes,
    which sends the mixed workload's 8198 rows down the block-major path."""
    scale_mode = syn.SCALE_PER_TOKEN_HEAD if name == "fp8_kv" else None
    _workload_parity(name, scale_mode, index_dtype, bench_workspace=True)


def _workload_parity(name, scale_mode, index_dtype, bench_workspace):
    b = _config(name, scale_mode, index_dtype)
    print(f"[workload] {name} scale_mode={scale_mode} index_dtype={index_dtype} rows={b.num_rows} "
          f"pages={b.num_pages} bench_workspace={bench_workspace}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    if bench_workspace:
        wsb = msa.msa_decode_workspace_bytes(b.num_rows, b.max_seq_len, b.num_q_heads, b.topk, 0)
        o.ws = torch.full((wsb // 4 + 1,), 0x3F3F3F3F, dtype=torch.int32, device="cuda")
        o.wsb = wsb
    H.run_decode(d, o)
    torch.cuda.synchronize()
    check_metadata(b, H.read_metadata(d))  # as written by the fused step itself
    scores = o.scores.cpu().numpy()
    table, ctx, sel = o.table.cpu().numpy(), o.ctx.cpu().numpy(), o.sel.cpu().numpy()
    out = H.bf16_to_np(o.out)
    # selection, tables and context lengths: every row, bit-exact on device scores
    check_selection(b, scores, table, ctx, sel, range(b.num_rows))
    rows = _sample_rows(b, 12 if b.num_rows <= 64 else 48, 7)
    ref_scores = check_scores(b, scores, rows)
    check_selection_valid(b, ref_scores, sel, rows)
    err = check_attention(b, out, table, ctx, rows)
    print(f"[workload] {name}: max attention err {err:.3e} over rows {rows[:8]}...", flush=True)
    # every row that selected anything produced a finite output
    assert np.isfinite(out).all()


@functools.lru_cache(maxsize=1)
def _most_requests_batch():
    return syn.random_batch(177, num_reqs=4096, max_len=130, topk=3)


@pytest.mark.parametrize("block_major", [False, True])
def test_fused_decode_most_requests(gpu_lib, block_major):
    """The most requests a batch may hold (4096), one row each, through the
    fused step: the metadata the score kernel writes, every row's selection,
    table and context length bit-exact; attention on sampled rows. With the
    larger workspace the 4096 rows take the block-major path."""
    b = _most_requests_batch()
    print(f"[fused] most requests rows={b.num_rows} block_major={block_major}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    if block_major:
        wsb = msa.msa_decode_workspace_bytes(b.num_rows, b.max_seq_len, b.num_q_heads, b.topk, 0)
        o.ws = torch.full((wsb // 4 + 1,), 0x3F3F3F3F, dtype=torch.int32, device="cuda")
        o.wsb = wsb
    H.run_decode(d, o)
    torch.cuda.synchronize()
    check_metadata(b, H.read_metadata(d))
    scores = o.scores.cpu().numpy()
    table, ctx, sel = o.table.cpu().numpy(), o.ctx.cpu().numpy(), o.sel.cpu().numpy()
    check_selection(b, scores, table, ctx, sel, range(b.num_rows))
    rows = _sample_rows(b, 16, 178)
    check_scores(b, scores, rows)
    out = H.bf16_to_np(o.out)
    assert np.isfinite(out).all()
    assert check_attention(b, out, table, ctx, rows) <= 2e-2

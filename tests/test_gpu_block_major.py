"""GPU parity of the block-major path of the fused step (launches of at
least 2048 rows given msa_decode_workspace_bytes): selections, tables and
context lengths bit-exact against the oracle selector on the device's scores;
attention (with LSE and sinks) against the oracle on the device's own table,
to the same bars as the per-row path; and the per-row path on the same
inputs (smaller workspace) within the same bars."""
import dataclasses

import numpy as np
import pytest
import torch

import block_sparse_paged_msa_amd as msa
import msa_synth as syn
from oracle import msa_oracle as O
from tests import bars
from tests import helpers as H
from tests.test_gpu_parity import check_metadata, check_scores, check_selection, _sample_rows

pytestmark = pytest.mark.gpu

ATOL = {syn.KV_BF16: 2e-2, syn.KV_FP8: 6e-2}
ATOL_LSE = 1e-3

CASES = [
    # (lengths, query rows, top-k, q heads, kv dtype, scale mode): prefill
    # requests among decode rows; short requests whose rows select one block
    # (their output is written by the block kernel itself); two head groups
    ([16384, 16384, 6000, 9000], [1, 1, 2100, 1000], 16, 16, syn.KV_BF16, syn.SCALE_NONE),
    ([100, 4000, 20000, 300], [100, 1800, 3, 250], 8, 16, syn.KV_FP8, syn.SCALE_PER_TOKEN_HEAD),
    ([3000, 12000], [1500, 600], 24, 24, syn.KV_FP8, syn.SCALE_SCALAR),
    # top-k 1: every row has a single slot, merged (normalised) by the merge kernel
    ([5000, 3000], [1500, 700], 1, 16, syn.KV_BF16, syn.SCALE_NONE),
    # bf16 K/V with per-token-head scales
    ([6000, 2500], [1400, 900], 12, 16, syn.KV_BF16, syn.SCALE_PER_TOKEN_HEAD),
    # requests with no query rows around a prefill request
    ([4000, 9000, 500, 7000], [0, 2100, 0, 0], 8, 16, syn.KV_BF16, syn.SCALE_NONE),
    # three head groups, the last one partial
    ([5000, 3000], [1300, 800], 8, 40, syn.KV_BF16, syn.SCALE_NONE),
    # more (request, block) pairs (40 x 469) than the launches that count
    # each block's rows and balance the grid by entries: blocks go to
    # workgroups by grid stride
    ([60000] + [2000 + 600 * i for i in range(39)], [2100] + [1] * 39, 16, 16, syn.KV_BF16, syn.SCALE_NONE),
    # a prefill request of 1094 blocks: the top-k's keys past the 1024 held in
    # registers, and 35 selection words per row
    ([140000, 3000, 500], [2100, 1, 1], 16, 16, syn.KV_BF16, syn.SCALE_NONE),
]


def _sinks(seed, hq):
    s = syn.SplitMix64(seed).uniform(hq) * 6.0 - 1.0
    s[0] = -np.inf
    return s.astype(np.float32)


@pytest.mark.parametrize("with_extras", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_block_major_step(gpu_lib, case, with_extras):
    L, ql, topk, hq, kv, sm = CASES[case]
    b = syn.make_batch("bm", 800 + case, L, ql, topk=topk, num_q_heads=hq, kv_dtype=kv, scale_mode=sm)
    assert b.num_rows >= 2048
    print(f"[block-major] case {case} rows={b.num_rows} extras={with_extras}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    wsb = msa.msa_decode_workspace_bytes(b.num_rows, b.max_seq_len, hq, topk, 0)
    assert wsb > o.wsb
    o.ws = torch.full((wsb // 4 + 1,), 0x3F3F3F3F, dtype=torch.int32, device="cuda")  # garbage on entry
    o.wsb = wsb
    sinks = _sinks(810 + case, hq) if with_extras else None
    lse = H.run_decode_lse(d, o, sinks)
    torch.cuda.synchronize()
    check_metadata(b, H.read_metadata(d))
    scores = o.scores.cpu().numpy()
    table, ctx, sel = o.table.cpu().numpy(), o.ctx.cpu().numpy(), o.sel.cpu().numpy()
    check_selection(b, scores, table, ctx, sel, range(b.num_rows))
    out = H.bf16_to_np(o.out)
    assert np.isfinite(out).all()
    rows = _sample_rows(b, 16, 820 + case)
    # rows whose selection is one block are written by the block kernel itself
    rows += [n for n in range(b.num_rows) if ctx[n] <= 128][:8]
    rows = sorted(set(rows))
    ref_out, ref_lse = O.attention_lse_from_table(b, table, ctx, rows, sinks)
    err = np.abs(out[rows] - ref_out).max()
    assert err <= ATOL[kv], f"attention max abs err {err}"
    _, amean = bars.oracle_and_abs_mean(b, table, ctx, rows)
    ex = bars.detect_excess(out[rows], ref_out, amean)
    assert ex <= 0, f"attention outside the detector bar by {ex} (max abs err {err})"
    lerr = np.abs(lse[rows] - ref_lse).max()
    assert lerr <= ATOL_LSE, f"lse max abs err {lerr}"
    # the per-row path on the same inputs (the smaller workspace selects it)
    o2 = H.alloc_decode(d)
    H.run_decode_lse(d, o2, sinks)
    assert torch.equal(o2.table, o.table) and torch.equal(o2.ctx, o.ctx)
    d_out = np.abs(H.bf16_to_np(o2.out) - out).max()
    assert d_out <= ATOL[kv], f"block-major vs per-row max abs diff {d_out}"


@pytest.mark.parametrize("sm_scale", [4.0, 1e-3])
def test_block_major_extreme_softmax_scale(gpu_lib, sm_scale):
    """Sharp and flat softmax through the block-major path with bf16 K/V and
    no scales (block partials scaled from the block's 128 max|V| bound): the
    same bars as the per-row path, and the per-row path agrees."""
    L, ql, topk, hq = [9000, 3000], [1800, 400], 16, 16
    b = syn.make_batch("bm_smscale", 880, L, ql, topk=topk, num_q_heads=hq, kv_dtype=syn.KV_BF16,
                       scale_mode=syn.SCALE_NONE)
    b = dataclasses.replace(b, sm_scale=sm_scale)
    print(f"[block-major] sm_scale={sm_scale} rows={b.num_rows}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    wsb = msa.msa_decode_workspace_bytes(b.num_rows, b.max_seq_len, hq, topk, 0)
    o.ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
    o.wsb = wsb
    H.run_decode(d, o)
    torch.cuda.synchronize()
    table, ctx = o.table.cpu().numpy(), o.ctx.cpu().numpy()
    out = H.bf16_to_np(o.out)
    assert np.isfinite(out).all()
    rows = sorted(set(_sample_rows(b, 16, 885)))
    ref_out, amean = bars.oracle_and_abs_mean(b, table, ctx, rows)
    err = np.abs(out[rows] - ref_out).max()
    assert err <= ATOL[syn.KV_BF16], f"attention max abs err {err}"
    ex = bars.detect_excess(out[rows], ref_out, amean)
    assert ex <= 0, f"attention outside the detector bar by {ex} (max abs err {err})"
    o2 = H.alloc_decode(d)
    H.run_decode(d, o2)
    assert torch.equal(o2.table, o.table)
    d_out = np.abs(H.bf16_to_np(o2.out) - out).max()
    assert d_out <= ATOL[syn.KV_BF16], f"block-major vs per-row max abs diff {d_out}"


@pytest.mark.parametrize("seed", range(6))
def test_block_major_random_batches(gpu_lib, seed):
    """Prefill-sized batches whose shape is drawn from the seed (one to three
    prefill requests of 700 to 2600 rows on contexts of up to 20000 tokens,
    up to eight decode or empty requests around them, top-k, query heads, K/V
    dtype and scale mode, index dtype) through the block-major path: selections, tables
    and context lengths bit-exact on every row, attention within the bars on
    sampled rows, and the per-row path agrees."""
    rng = syn.SplitMix64(7100 + seed)
    npf, nd = int(rng.integers(1, 3, 1)[0]), int(rng.integers(0, 8, 1)[0])
    qpf = rng.integers(700, 2600, npf)
    Lpf = qpf + rng.integers(0, 17400, npf)
    Ld = np.where(rng.uniform(nd) < 0.25, 0, rng.integers(1, 20000, nd))
    L = np.concatenate([Ld, Lpf]).astype(np.int64)
    ql = np.concatenate([np.minimum(Ld, 1), qpf]).astype(np.int64)
    if ql.sum() < 2048:
        ql[-1] += 2048 - ql.sum()
        L[-1] = max(L[-1], ql[-1])
    pick = lambda opts: opts[int(rng.integers(0, len(opts) - 1, 1)[0])]
    topk, hq = pick([1, 4, 16, 32]), pick([16, 24, 32])
    kv, sm = pick([(syn.KV_BF16, syn.SCALE_NONE), (syn.KV_BF16, syn.SCALE_PER_TOKEN_HEAD),
                   (syn.KV_FP8, syn.SCALE_SCALAR), (syn.KV_FP8, syn.SCALE_PER_TOKEN_HEAD)])
    idx = pick([syn.INDEX_BF16, syn.INDEX_FP8])
    b = syn.make_batch("bm_random", 7100 + seed, L, ql, topk=topk, num_q_heads=hq, kv_dtype=kv, scale_mode=sm,
                       index_dtype=idx)
    assert b.num_rows >= 2048
    print(f"[block-major] random seed {seed}: L={L.tolist()} ql={ql.tolist()} topk={topk} hq={hq} kv={kv} "
          f"scale={sm} index={idx}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    wsb = msa.msa_decode_workspace_bytes(b.num_rows, b.max_seq_len, hq, topk, 0)
    o.ws = torch.full((wsb // 4 + 1,), 0x3F3F3F3F, dtype=torch.int32, device="cuda")
    o.wsb = wsb
    H.run_decode(d, o)
    torch.cuda.synchronize()
    check_metadata(b, H.read_metadata(d))
    scores = o.scores.cpu().numpy()
    table, ctx, sel = o.table.cpu().numpy(), o.ctx.cpu().numpy(), o.sel.cpu().numpy()
    check_selection(b, scores, table, ctx, sel, range(b.num_rows))
    out = H.bf16_to_np(o.out)
    assert np.isfinite(out).all()
    rows = _sample_rows(b, 16, 7150 + seed)
    rows = sorted(set(rows + [n for n in range(b.num_rows) if ctx[n] <= 128][:8]))
    ref, amean = bars.oracle_and_abs_mean(b, table, ctx, rows)
    err = np.abs(out[rows] - ref).max()
    assert err <= ATOL[kv], f"attention max abs err {err}"
    ex = bars.detect_excess(out[rows], ref, amean)
    assert ex <= 0, f"attention outside the detector bar by {ex} (max abs err {err})"
    o2 = H.alloc_decode(d)
    H.run_decode(d, o2)
    assert torch.equal(o2.table, o.table) and torch.equal(o2.ctx, o.ctx)
    assert np.abs(H.bf16_to_np(o2.out) - out).max() <= ATOL[kv]


@pytest.mark.parametrize("vexp", [40, -60])
def test_block_major_extreme_values(gpu_lib, vexp):
    """V scaled by 2^vexp (exact in bf16): the fp16 block partials are scaled
    by a power of two chosen from their own magnitude, so the outputs scale
    with V and stay within the bars relative to it."""
    L, ql, topk, hq = [9000, 3000], [1800, 400], 16, 16
    b = syn.make_batch("bm_scale", 830 + (vexp & 7), L, ql, topk=topk, num_q_heads=hq,
                       kv_dtype=syn.KV_BF16, scale_mode=syn.SCALE_NONE)
    f = (b.v_cache.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** vexp)
    b.v_cache = (f.view(np.uint32) >> 16).astype(np.uint16)
    print(f"[block-major] V x 2^{vexp} rows={b.num_rows}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    wsb = msa.msa_decode_workspace_bytes(b.num_rows, b.max_seq_len, hq, topk, 0)
    o.ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
    o.wsb = wsb
    H.run_decode(d, o)
    torch.cuda.synchronize()
    table, ctx = o.table.cpu().numpy(), o.ctx.cpu().numpy()
    out = H.bf16_to_np(o.out)
    assert np.isfinite(out).all()
    rows = sorted(set(_sample_rows(b, 16, 840)))
    ref = O.attention_from_table(b, table, ctx, rows)
    err = np.abs(out[rows] - ref).max() / 2.0 ** vexp
    assert err <= ATOL[syn.KV_BF16], f"attention max abs err {err} (in units of 2^{vexp})"


@pytest.mark.parametrize("outlier", [2.0 ** 12, 2.0 ** 16])
def test_block_major_value_outlier(gpu_lib, outlier):
    """One token with |V| = outlier in every dim, in the block that most rows
    of the prefill request keep: every row that attends that block, whatever
    weight it gives the outlier, stays within the detector bar (the fp16 block
    partials must not lose the small accumulators of those rows)."""
    L, ql, topk, hq = [9000, 3000], [2000, 300], 16, 16
    b = syn.make_batch("bm_outlier", 860, L, ql, topk=topk, num_q_heads=hq, kv_dtype=syn.KV_BF16,
                       scale_mode=syn.SCALE_NONE)
    d = H.upload(b)
    o = H.alloc_decode(d)
    wsb = msa.msa_decode_workspace_bytes(b.num_rows, b.max_seq_len, hq, topk, 0)
    o.ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
    o.wsb = wsb
    H.run_decode(d, o)                       # the selection does not depend on V
    torch.cuda.synchronize()
    sel = o.sel.cpu().numpy()[:2000]
    counts = np.bincount(sel[sel >= 0], minlength=b.ld_s)
    blk = int(np.argmax(counts[:(9000 - 2000) // 128]))   # a block every row sees whole
    page = int(b.block_table[0, blk])
    tok = 77                                  # token 77 of the block: sub-page 4, slot 13
    sub, slot = 8 * page + tok // 16, tok % 16
    signs = np.where(syn.SplitMix64(861).uniform(128) < 0.5, -outlier, outlier)
    b.v_cache[sub, 0, :, slot] = syn.to_bf16_bits(signs)
    print(f"[block-major] |V| outlier {outlier} in block {blk}, kept by {counts[blk]} of 2000 rows", flush=True)
    d = H.upload(b)
    H.run_decode(d, o)
    torch.cuda.synchronize()
    table, ctx = o.table.cpu().numpy(), o.ctx.cpu().numpy()
    out = H.bf16_to_np(o.out)
    assert np.isfinite(out).all()
    rows = [n for n in range(2000) if blk in sel[n]][:40] + sorted(set(_sample_rows(b, 8, 862)))
    ref, amean = bars.oracle_and_abs_mean(b, table, ctx, rows)
    ex = bars.detect_excess(out[rows], ref, amean)
    assert ex <= 0, f"outside the detector bar by {ex} (max abs err {np.abs(out[rows] - ref).max()})"


def test_block_major_scores_in_workspace(gpu_lib):
    """No caller score buffer: the block-major workspace also holds the
    scores (ld_s > 0 in msa_decode_workspace_bytes); same outputs, tables and
    context lengths as with a caller buffer."""
    L, ql, topk, hq = [7000, 5000, 300], [1200, 900, 1], 8, 16
    b = syn.make_batch("bm_ws", 850, L, ql, topk=topk, num_q_heads=hq, kv_dtype=syn.KV_BF16,
                       scale_mode=syn.SCALE_NONE)
    print(f"[block-major] scores in workspace rows={b.num_rows}", flush=True)
    d = H.upload(b)
    outs = []
    for with_scores in (True, False):
        o = H.alloc_decode(d)
        wsb = msa.msa_decode_workspace_bytes(b.num_rows, b.max_seq_len, hq, topk, 0 if with_scores else b.ld_s)
        o.ws = torch.full((wsb // 4 + 1,), 0x3F3F3F3F, dtype=torch.int32, device="cuda")
        o.wsb = wsb
        H.run_decode(d, o, with_scores=with_scores)
        torch.cuda.synchronize()
        outs.append(o)
    assert torch.equal(outs[0].table, outs[1].table) and torch.equal(outs[0].ctx, outs[1].ctx)
    assert torch.equal(outs[0].out, outs[1].out)
    ctx = outs[0].ctx.cpu().numpy()
    rows = sorted(set(_sample_rows(b, 12, 851)))
    ref = O.attention_from_table(b, outs[0].table.cpu().numpy(), ctx, rows)
    err = np.abs(H.bf16_to_np(outs[1].out)[rows] - ref).max()
    assert err <= ATOL[syn.KV_BF16], f"attention max abs err {err}"


def test_block_major_repeat_and_graph_replay_bitwise(gpu_lib):
    """The block-major step is deterministic (every (row, block) entry writes
    its own slot; the merge takes slots in rank order), and a captured step
    replays bit for bit with garbage left in the workspace between replays."""
    b = syn.make_batch("bm_graph", 860, [9000, 20000, 700], [1600, 600, 1], topk=16, num_q_heads=16,
                       kv_dtype=syn.KV_FP8, scale_mode=syn.SCALE_PER_TOKEN_HEAD)
    print(f"[block-major] graph replay rows={b.num_rows}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    wsb = msa.msa_decode_workspace_bytes(b.num_rows, b.max_seq_len, 16, b.topk, 0)
    o.ws = torch.full((wsb // 4 + 1,), 0x3F3F3F3F, dtype=torch.int32, device="cuda")
    o.wsb = wsb
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
        H.run_decode(d, o)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        H.run_decode(d, o)
    for rep in range(3):
        o.out.zero_()
        o.table.fill_(-1)
        o.ws.fill_(0x3F3F3F3F)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip((o.out, o.table, o.ctx, o.sel, o.scores), ref):
            assert torch.equal(t, r), f"replay {rep}"


@pytest.mark.parametrize("topk", [1, 8, 16])
def test_block_major_tied_scores(gpu_lib, topk):
    """Index queries and keys in {-1, 0, 1}: integer token scores, so many
    blocks share their pooled maximum and the cut falls inside a tie (the
    lowest block ids are kept); the selection words the top-k step leaves
    for the block kernel carry the same choice as the oracle's, and the
    per-row path on the same inputs gives the same table."""
    L, ql = [9000, 5000, 300, 2047], [1500, 700, 1, 1]
    b = syn.make_batch("bm_ties", 870 + topk, L, ql, topk=topk, num_q_heads=16, kv_dtype=syn.KV_BF16,
                       scale_mode=syn.SCALE_NONE)
    tern = lambda x: syn.to_bf16_bits(np.clip(np.round(O.bf16_to_f64(x)), -1.0, 1.0))
    b = dataclasses.replace(b, index_q=tern(b.index_q), index_k=tern(b.index_k))
    assert b.num_rows >= 2048
    print(f"[block-major] ties topk={topk} rows={b.num_rows}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    wsb = msa.msa_decode_workspace_bytes(b.num_rows, b.max_seq_len, 16, topk, 0)
    o.ws = torch.full((wsb // 4 + 1,), 0x3F3F3F3F, dtype=torch.int32, device="cuda")
    o.wsb = wsb
    H.run_decode(d, o)
    torch.cuda.synchronize()
    scores = o.scores.cpu().numpy()
    table, ctx, sel = o.table.cpu().numpy(), o.ctx.cpu().numpy(), o.sel.cpu().numpy()
    meta = O.build_metadata(b.seq_lens, b.query_lens)
    straddled = 0
    for n in range(b.num_rows):
        nb = O.num_blocks(O.visible_keys(meta["row_pos"][n]))
        row = scores[n][:nb].astype(np.float64)
        assert np.array_equal(row, np.round(row)), f"row {n}: scores are not integers"
        if topk < nb:
            srt = np.sort(row)[::-1]
            straddled += int(srt[topk - 1] == srt[topk])
    assert straddled >= 1, "the crafted inputs should put the cut inside a tie"
    check_selection(b, scores, table, ctx, sel, range(b.num_rows))
    rows = sorted(set(_sample_rows(b, 12, 880 + topk)))
    check_scores(b, scores, rows)
    ref = O.attention_from_table(b, table, ctx, rows)
    err = np.abs(H.bf16_to_np(o.out)[rows] - ref).max()
    assert err <= ATOL[syn.KV_BF16], f"attention max abs err {err}"
    o2 = H.alloc_decode(d)
    H.run_decode(d, o2)
    assert torch.equal(o2.table, o.table) and torch.equal(o2.ctx, o.ctx)

"""GPU parity of the natural-log LSE output and the per-head sinks
(msa_sparse_paged_attn_ex / msa_sparse_decode_ex through the C ABI) with the
oracle run on the device's own table and context lengths.

Bars: outputs as for plain attention (2e-2 absolute for bf16 K/V, 6e-2 for
fp8); LSE within 1e-3 absolute. The LSE bar: logits come from exact bf16 or
widened-fp8 products summed in fp32 (relative error about 1e-5 of
sum |q k| * sm_scale, a few units here), and the denominator is an fp32 sum of
at most 38400 exponentials from the hardware exp2 (relative error ~1e-5), so
the error stays near 1e-4; rows with nothing to attend give exactly -inf."""
import numpy as np
import pytest
import torch

import msa_synth as syn
from oracle import msa_oracle as O
from tests import bars
from tests import helpers as H

pytestmark = pytest.mark.gpu

ATOL_BF16 = 2e-2
ATOL_FP8 = 6e-2
ATOL_LSE = 1e-3


def _sinks(seed, hq):
    s = syn.SplitMix64(seed).uniform(hq) * 8.0 - 2.0
    s[1] = -np.inf                                   # a head with no sink
    return s.astype(np.float32)


def _check(b, out, lse, table, ctx, rows, sinks):
    ref_out, ref_lse = O.attention_lse_from_table(b, table, ctx, rows, sinks)
    atol = ATOL_FP8 if b.kv_dtype == syn.KV_FP8 else ATOL_BF16
    err = np.abs(out[rows] - ref_out).max()
    assert err <= atol, f"output max abs err {err}"
    _, amean = bars.oracle_and_abs_mean(b, table, ctx, rows)
    ex = bars.detect_excess(out[rows], ref_out, amean)
    assert ex <= 0, f"output outside the detector bar by {ex} (max abs err {err})"
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse[rows]), empty), "-inf LSE exactly for rows with nothing to attend"
    lerr = np.abs(lse[rows][~empty] - ref_lse[~empty]).max(initial=0.0)
    assert lerr <= ATOL_LSE, f"lse max abs err {lerr}"


CASES = [
    dict(kv=syn.KV_BF16, sm=syn.SCALE_NONE, hq=16),
    dict(kv=syn.KV_BF16, sm=syn.SCALE_NONE, hq=24),
    dict(kv=syn.KV_FP8, sm=syn.SCALE_SCALAR, hq=8),
    dict(kv=syn.KV_FP8, sm=syn.SCALE_PER_TOKEN_HEAD, hq=16),
]


@pytest.mark.parametrize("with_sinks", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_attention_lse_on_device_table(gpu_lib, case, with_sinks):
    c = CASES[case]
    b = syn.make_batch("lse", 500 + case, [9000, 700, 129, 1, 20000, 3000], [1, 2, 1, 1, 1, 3], topk=24,
                       num_q_heads=c["hq"], kv_dtype=c["kv"], scale_mode=c["sm"])
    print(f"[lse] table case={c} sinks={with_sinks}", flush=True)
    d = H.upload(b)
    H.run_metadata(d)
    table, ctx, _ = H.run_topk(d, H.run_scores(d))
    ctx[2] = 0                                      # a row with nothing to attend
    sinks = _sinks(510 + case, b.num_q_heads) if with_sinks else None
    out, lse = H.run_attn_lse(d, table, ctx, sinks, max_ctx=128 * b.topk)
    rows = list(range(b.num_rows))
    _check(b, out, lse, table, ctx, rows, sinks)
    if not with_sinks:   # the plain entry point is this one with no extras: same bits
        assert np.array_equal(H.run_attn(d, table, ctx, max_ctx=128 * b.topk), out)


FUSED = [
    # (name, lengths, query rows, top-k, query heads, kv dtype, scale mode)
    ("mix", [9000, 0, 700, 129, 300, 1], [1, 0, 2, 0, 3, 1], 16, 16, syn.KV_BF16, syn.SCALE_NONE),
    ("topk300", [140000, 70000], [1, 2], 300, 16, syn.KV_BF16, syn.SCALE_NONE),   # the merge kernel
    ("hq24fp8", [9000, 3000, 20000], [1, 3, 2], 24, 24, syn.KV_FP8, syn.SCALE_PER_TOKEN_HEAD),
    ("coop", [120000, 50000], [1, 1], 64, 16, syn.KV_FP8, syn.SCALE_SCALAR),       # 257..1024 blocks
]


@pytest.mark.parametrize("case", range(len(FUSED)))
def test_fused_decode_lse_and_sinks(gpu_lib, case):
    name, L, ql, topk, hq, kv, sm = FUSED[case]
    b = syn.make_batch(name, 520 + case, L, ql, topk=topk, num_q_heads=hq, kv_dtype=kv, scale_mode=sm)
    print(f"[lse] fused {name} rows={b.num_rows} topk={topk} hq={hq}", flush=True)
    d = H.upload(b)
    rows = list(range(b.num_rows))
    o0 = H.alloc_decode(d)
    H.run_decode(d, o0)
    o1 = H.alloc_decode(d)
    lse1 = H.run_decode_lse(d, o1, None)
    assert torch.equal(o1.out, o0.out) and torch.equal(o1.table, o0.table)   # no sinks: same bits
    sinks = _sinks(530 + case, hq)
    o2 = H.alloc_decode(d)
    lse2 = H.run_decode_lse(d, o2, sinks)
    assert np.array_equal(lse2, lse1)                # the LSE leaves the sink out
    table, ctx = o2.table.cpu().numpy(), o2.ctx.cpu().numpy()
    _check(b, H.bf16_to_np(o2.out), lse2, table, ctx, rows, sinks)


def test_lse_merges_two_halves_of_a_row(gpu_lib):
    """Context-parallel use: attention over the first and the second half of
    every row's tokens, merged on the host with the two LSEs, matches the
    attention over all tokens; the merged LSE matches the whole one."""
    b = syn.make_batch("lsecp", 540, [40000, 9000, 3000], [1, 2, 1], topk=32, num_q_heads=16,
                       kv_dtype=syn.KV_FP8, scale_mode=syn.SCALE_PER_TOKEN_HEAD)
    d = H.upload(b)
    H.run_metadata(d)
    table, ctx, _ = H.run_topk(d, H.run_scores(d))
    out, lse = H.run_attn_lse(d, table, ctx, None, max_ctx=128 * b.topk)
    half = 8 * (b.topk // 2)                         # sub-pages in the first half
    ctx_a = np.minimum(ctx, 16 * half)
    ctx_b = ctx - ctx_a
    table_b = np.zeros_like(table)
    table_b[:, :table.shape[1] - half] = table[:, half:]
    out_a, lse_a = H.run_attn_lse(d, table, ctx_a, None, max_ctx=128 * b.topk)
    out_b, lse_b = H.run_attn_lse(d, table_b, ctx_b, None, max_ctx=128 * b.topk)
    lse_m = np.logaddexp(lse_a, lse_b)
    wa = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - lse_m))
    wb = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - lse_m))
    merged = out_a * wa[..., None] + out_b * wb[..., None]
    assert np.abs(lse_m - lse).max() <= ATOL_LSE
    assert np.abs(merged - out).max() <= ATOL_FP8


def test_extreme_sinks(gpu_lib):
    """A sink far above every logit (or +inf) leaves zeros; the LSE is unchanged."""
    b = syn.make_batch("lsex", 550, [5000, 200], [1, 1], topk=8, num_q_heads=16)
    d = H.upload(b)
    H.run_metadata(d)
    table, ctx, _ = H.run_topk(d, H.run_scores(d))
    _, lse0 = H.run_attn_lse(d, table, ctx, None, max_ctx=128 * b.topk)
    sinks = np.full(16, 1e4, np.float32)
    sinks[3] = np.inf
    out, lse = H.run_attn_lse(d, table, ctx, sinks, max_ctx=128 * b.topk)
    assert np.all(out == 0.0) and np.array_equal(lse, lse0)

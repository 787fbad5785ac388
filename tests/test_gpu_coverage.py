"""Every attended token counted exactly once, on every row of full-size
workloads.

With a zero query every logit is 0, so each (row, head)'s softmax is uniform
over the row's ctx tokens: the probabilities are exactly 1, the denominator is
exactly ctx in fp32 (an integer below 2^24), so exp(lse) = ctx, and the output
is the mean of the dequantised values over the tokens the page-16 table names.
One selected block dropped or attended twice moves the count by up to 128 and
the mean far beyond its bar (tests/test_bars_cpu.py shows both on the CPU).
This is the check the split-K ragged-tail bug class calls for (vLLM PR #54404
page, 关键源码片段: a kernel that mishandles ragged tails with split KV).

The expected mean is the closed form of the oracle's attention at q = 0
(pinned in tests/test_oracle_pins.py); a few rows are also run through the
oracle itself. Per-token-head V scales are rounded to bf16 values first, so
that the product of a probability of 1 with its scale is exact in the bf16
operand the PV products take; the count check does not depend on it.
"""
import dataclasses
import functools

import numpy as np
import pytest
import torch

import block_sparse_paged_msa_amd as msa
import msa_synth as syn
from oracle import msa_oracle as O
from tests import bars
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _value_means(b, table, ctx, rows):
    """Mean over tokens u < ctx[n] of the dequantised V row of token u, the
    token walked through the page-16 table (entry u // 16, slot u % 16)."""
    dec = O.bf16_to_f64 if b.kv_dtype == syn.KV_BF16 else O.e4m3fn_to_f64
    nsub = (ctx[rows] + 15) // 16
    used = np.unique(np.concatenate([table[n, :k] for n, k in zip(rows, nsub)] + [np.zeros(1, table.dtype)]))
    vals = dec(b.v_cache[used, 0])                              # [U][128 dims][16 slots]
    if b.scale_mode == syn.SCALE_PER_TOKEN_HEAD:
        vals = vals * b.v_scale[used, :, 0].astype(np.float64)[:, None, :]
    elif b.scale_mode == syn.SCALE_SCALAR:
        vals = vals * float(b.v_scale.reshape(-1)[0])
    cum = np.concatenate([np.zeros(vals.shape[:2] + (1,)), np.cumsum(vals, axis=2)], axis=2)
    out = np.zeros((len(rows), 128))
    for i, n in enumerate(rows):
        c = int(ctx[n])
        if c == 0:
            continue
        full, rem = divmod(c, 16)
        idx = np.searchsorted(used, table[n, :full])
        s = cum[idx, :, 16].sum(axis=0)
        if rem:
            s = s + cum[np.searchsorted(used, table[n, full]), :, rem]
        out[i] = s / c
    return out


def _zero_query(b):
    bz = dataclasses.replace(b, q=np.zeros_like(b.q))
    if b.scale_mode == syn.SCALE_PER_TOKEN_HEAD:
        vs = O.bf16_to_f64(syn.to_bf16_bits(b.v_scale.astype(np.float64))).astype(np.float32)
        bz = dataclasses.replace(bz, v_scale=vs)
    return bz


@functools.lru_cache(maxsize=1)
def _batch(name, scale_mode):
    if name == "topk300":
        return syn.make_batch("topk300", 140, [140000, 70000], [1, 2], topk=300, num_q_heads=16)
    return syn.config(name, scale_mode=scale_mode)


def _check_coverage(b, out, lse, table, ctx, rows, tag):
    cnt = np.rint(np.exp(lse[rows]))
    bad = np.argwhere(cnt != ctx[rows][:, None].astype(np.float64))
    assert bad.size == 0, f"{tag}: exp(lse) != ctx at (row, head) {bad[:5].tolist()} " \
                          f"(got {cnt[tuple(bad[0])]}, ctx {ctx[rows][bad[0][0]]})"
    rel = np.abs(np.exp(lse[rows]) / ctx[rows][:, None] - 1.0).max()
    assert rel <= 1e-5, f"{tag}: exp(lse) / ctx - 1 = {rel}"
    mean = _value_means(b, table, ctx, rows)
    ex = bars.cover_excess(out[rows], mean[:, None, :])
    print(f"[coverage] {tag}: {len(rows)} rows, ctx {int(ctx.min())}..{int(ctx.max())}, "
          f"max |out - mean| {np.abs(out[rows] - mean[:, None, :]).max():.2e}, bar excess {ex:.2e}", flush=True)
    assert ex <= 0, f"{tag}: output off the mean of the attended values by {ex} beyond the bar"


@pytest.mark.parametrize("name,scale_mode,block_major", [
    ("bf16_batch", None, False),
    ("spec_decode", None, False),
    ("fp8_kv", syn.SCALE_PER_TOKEN_HEAD, False),
    ("fp8_kv", syn.SCALE_SCALAR, False),
    ("topk300", None, False),
    ("mixed_prefill", None, True),
])
def test_zero_query_counts_every_token_once(gpu_lib, name, scale_mode, block_major):
    b = _zero_query(_batch(name, scale_mode))
    print(f"[coverage] {name} scale_mode={scale_mode} rows={b.num_rows} block_major={block_major}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    if block_major:
        wsb = msa.msa_decode_workspace_bytes(b.num_rows, b.max_seq_len, b.num_q_heads, b.topk, 0)
        o.ws = torch.full((wsb // 4 + 1,), 0x3F3F3F3F, dtype=torch.int32, device="cuda")
        o.wsb = wsb
    lse = H.run_decode_lse(d, o, None)
    torch.cuda.synchronize()
    table, ctx = o.table.cpu().numpy(), o.ctx.cpu().numpy()
    out = H.bf16_to_np(o.out)
    rows = list(range(b.num_rows))
    assert ctx.min() > 0
    _check_coverage(b, out, lse, table, ctx, rows, name)
    # the oracle itself on a few rows agrees with the closed form
    some = rows[:2] + rows[-1:]
    ref_out, ref_lse = O.attention_lse_from_table(b, table, ctx, some)
    assert np.allclose(ref_lse, np.log(ctx[some].astype(np.float64))[:, None], rtol=0, atol=1e-12)
    assert bars.cover_excess(ref_out, _value_means(b, table, ctx, some)[:, None, :]) <= -bars.COVER_ATOL / 2
    # the table-driven entry point on the device's own table counts the same
    if not block_major:
        out2, lse2 = H.run_attn_lse(d, table, ctx, None, max_ctx=128 * b.topk)
        _check_coverage(b, out2, lse2, table, ctx, rows, name + " (table entry)")

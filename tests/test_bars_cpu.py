"""The attention bars can fail: on full-size rows of the bf16 batch and the
fp8 K/V workloads, the oracle's own output with one selected block dropped,
or with one block attended twice in place of another, lies outside the
detector bar (tests/bars.py), and with a zero query the softmax denominator
no longer equals the row's context length. This is what the GPU coverage and
detector checks rely on to see a ragged-tail or split-edge mistake."""
import functools

import numpy as np
import pytest

import msa_synth as syn
from oracle import msa_oracle as O
from tests import bars


@functools.lru_cache(maxsize=None)
def _row0(name):
    scale_mode = syn.SCALE_PER_TOKEN_HEAD if name == "fp8_kv" else None
    b = syn.config(name, scale_mode=scale_mode)
    res = O.decode_step(b, rows=[0])
    _, amean = bars.oracle_and_abs_mean(b, res["table"], res["ctx"], [0])
    return b, res["table"], res["ctx"], res["sel"][0], res["out"][0], amean[0]


def _drop_block(table, ctx, sel, n, j, v):
    """Row n's table without its j-th selected block: later entries move up
    eight places, the context loses that block's visible tokens."""
    t, c = table.copy(), ctx.copy()
    row = t[n].tolist()
    del row[8 * j:8 * j + 8]
    t[n] = row + [0] * 8
    c[n] -= min(128, v - 128 * int(sel[j]))
    return t, c


@pytest.mark.parametrize("name", ["bf16_batch", "fp8_kv"])
def test_dropped_or_doubled_block_fails_the_detector_bar(name):
    b, table, ctx, sel, ref, amean = _row0(name)
    kk = int((sel >= 0).sum())
    v = int(b.seq_lens[0])              # one row per request: the row sees L keys
    assert np.allclose(O.attention_from_table(b, table, ctx, [0])[0], ref, rtol=0, atol=1e-12)
    missed_by_contract = 0
    for j in sorted({0, kk // 2, kk - 2, kk - 1}):
        t, c = _drop_block(table, ctx, sel, 0, j, v)
        out = O.attention_from_table(b, t, c, [0])[0]
        assert bars.detect_excess(out, ref, amean) > 0, f"dropping selected block {j} went unseen"
        missed_by_contract += int(np.abs(out - ref).max() <= bars.contract_atol(b.kv_dtype))
    # one full block attended twice, in place of another full block
    t = table.copy()
    t[0, 8:16] = t[0, 0:8]
    out = O.attention_from_table(b, t, ctx, [0])[0]
    assert bars.detect_excess(out, ref, amean) > 0, "a doubled block went unseen"
    if name == "fp8_kv":
        # on the long fp8 rows the contract bar alone misses dropped blocks
        # (why the detector exists)
        assert missed_by_contract >= 1


def test_dropped_subpage_fails_the_detector_bar():
    """A single 16-token sub-page missing from the bf16 batch row."""
    b, table, ctx, sel, ref, amean = _row0("bf16_batch")
    t, c = table.copy(), ctx.copy()
    row = t[0].tolist()
    del row[3]
    t[0] = row + [0]
    c[0] -= 16
    out = O.attention_from_table(b, t, c, [0])[0]
    assert bars.detect_excess(out, ref, amean) > 0


@pytest.mark.parametrize("name", ["bf16_batch", "fp8_kv"])
def test_zero_query_counts_tokens_and_sees_a_dropped_block(name):
    """q = 0: exp(lse) equals the context length and the output is the mean
    of the attended values; one block fewer changes both beyond their bars."""
    b, table, ctx, sel, _, _ = _row0(name)
    bz = syn.Batch(**{**b.__dict__, "q": np.zeros_like(b.q)})
    out, lse = O.attention_lse_from_table(bz, table, ctx, [0])
    assert np.all(np.rint(np.exp(lse[0])) == ctx[0])
    _, vh = O._table_keys_values(bz, table, 0, int(ctx[0]), 0)
    mean = vh.mean(axis=0)
    assert bars.cover_excess(out[0], mean[None, :]) <= 0
    v = int(b.seq_lens[0])
    kk = int((sel >= 0).sum())
    t, c = _drop_block(table, ctx, sel, 0, kk // 2, v)
    out2, lse2 = O.attention_lse_from_table(bz, t, c, [0])
    assert np.all(np.rint(np.exp(lse2[0])) == c[0]) and c[0] != ctx[0]
    assert bars.cover_excess(out2[0], mean[None, :]) > 0

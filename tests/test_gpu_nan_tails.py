"""GPU: cache slots past a request's last token may hold anything, NaN
included (a page is allocated whole, only its first tokens are written). With
NaN planted in every such slot (index keys and their fp8 scales, K, V and
per-token-head scales), the fused step on the per-row and on the block-major
path must give finite outputs and the same scores, selections and attention
as the oracle, which never reads those slots."""
import numpy as np
import pytest
import torch

import block_sparse_paged_msa_amd as msa
import msa_synth as syn
from oracle import msa_oracle as O
from tests import bars
from tests import helpers as H
from tests.test_gpu_parity import check_scores, check_selection, _sample_rows

pytestmark = pytest.mark.gpu

ATOL = {syn.KV_BF16: 2e-2, syn.KV_FP8: 6e-2}

CASES = [
    # (lengths (none a multiple of 128), query rows, top-k, kv dtype, scale mode, index dtype)
    ([3000, 777, 12345, 200], [1, 1, 1, 1], 8, syn.KV_BF16, syn.SCALE_NONE, syn.INDEX_BF16),
    ([5001, 913, 20000 - 3], [2, 1, 3], 16, syn.KV_FP8, syn.SCALE_PER_TOKEN_HEAD, syn.INDEX_FP8),
    ([6100, 2900, 333], [1500, 700, 1], 16, syn.KV_BF16, syn.SCALE_PER_TOKEN_HEAD, syn.INDEX_BF16),
    ([4500, 3100], [1300, 900], 8, syn.KV_FP8, syn.SCALE_PER_TOKEN_HEAD, syn.INDEX_FP8),
    # block-major with no K/V scales and with a scalar pair
    ([7000, 2500, 90], [1400, 800, 1], 8, syn.KV_BF16, syn.SCALE_NONE, syn.INDEX_BF16),
    ([5100, 2300], [1200, 1000], 12, syn.KV_FP8, syn.SCALE_SCALAR, syn.INDEX_BF16),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_nan_in_unused_slots(gpu_lib, case):
    L, ql, topk, kv, sm, idx = CASES[case]
    b = syn.make_batch("nan", 870 + case, L, ql, topk=topk, num_q_heads=16, kv_dtype=kv, scale_mode=sm,
                       index_dtype=idx)
    planted = H.plant_nan_tails(b)
    assert planted > 0
    block_major = b.num_rows >= 2048
    print(f"[nan tails] case {case} rows={b.num_rows} planted={planted} block_major={block_major}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    if block_major:
        wsb = msa.msa_decode_workspace_bytes(b.num_rows, b.max_seq_len, 16, topk, 0)
        o.ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
        o.wsb = wsb
    H.run_decode(d, o)
    torch.cuda.synchronize()
    rows = sorted(set(_sample_rows(b, 12, 880 + case)))
    scores = o.scores.cpu().numpy()
    check_scores(b, scores, rows)
    table, ctx, sel = o.table.cpu().numpy(), o.ctx.cpu().numpy(), o.sel.cpu().numpy()
    check_selection(b, scores, table, ctx, sel, rows)
    out = H.bf16_to_np(o.out)
    assert np.isfinite(out).all(), "non-finite output"
    ref, amean = bars.oracle_and_abs_mean(b, table, ctx, rows)
    err = np.abs(out[rows] - ref).max()
    assert err <= ATOL[kv], f"attention max abs err {err}"
    assert bars.detect_excess(out[rows], ref, amean) <= 0, f"attention outside the detector bar (max abs err {err})"


@pytest.mark.parametrize("kv,sm", [(syn.KV_BF16, syn.SCALE_PER_TOKEN_HEAD), (syn.KV_FP8, syn.SCALE_PER_TOKEN_HEAD),
                                   (syn.KV_FP8, syn.SCALE_SCALAR)])
def test_nan_in_unused_slots_table_mode(gpu_lib, kv, sm):
    """msa_sparse_paged_attn on the oracle's own table and context lengths,
    with NaN in every slot past each request's last token."""
    b = syn.make_batch("nan_tab", 890 + kv + 2 * sm, [3001, 17777, 129], [1, 2, 1], topk=16, num_q_heads=16,
                       kv_dtype=kv, scale_mode=sm)
    H.plant_nan_tails(b)
    print(f"[nan tails] table mode kv={kv} scale_mode={sm} rows={b.num_rows}", flush=True)
    d = H.upload(b)
    ref = O.decode_step(b)
    out = H.run_attn(d, ref["table"], ref["ctx"])
    torch.cuda.synchronize()
    assert np.isfinite(out).all(), "non-finite output"
    err = np.abs(out - ref["out"]).max()
    assert err <= ATOL[kv], f"attention max abs err {err}"
    _, amean = bars.oracle_and_abs_mean(b, ref["table"], ref["ctx"], list(range(b.num_rows)))
    assert bars.detect_excess(out, ref["out"], amean) <= 0, f"attention outside the detector bar (max abs err {err})"

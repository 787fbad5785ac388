"""GPU parity of the prefill score tile (requests with more than 64 query
rows: 512 rows x 8 index-K pages per workgroup) through the C ABI: every row's
pooled scores against the oracle, and bit for bit against the per-row unit
scorer on the same rows presented as one-row requests."""
import numpy as np
import pytest
import torch

import block_sparse_paged_msa_amd as msa
import msa_synth as syn
from tests import helpers as H
from tests.test_gpu_parity import check_scores

pytestmark = pytest.mark.gpu

CASES = [
    # (lengths, query rows): a fresh prompt (rows from position 0, so most
    # pages are past most rows), 65 rows (one more than the unit scorer's
    # group), exactly one 256-row block, a partial last block, small requests
    ([1000, 3000, 5000, 2048, 700, 9000], [1000, 65, 1, 256, 64, 300]),
    ([130, 20000], [130, 513]),
]


@pytest.mark.parametrize("index_dtype", [syn.INDEX_BF16, syn.INDEX_FP8])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_tile_scores_every_row(gpu_lib, case, index_dtype):
    L, ql = CASES[case]
    b = syn.make_batch("tile", 700 + case, L, ql, topk=8, num_q_heads=16, index_dtype=index_dtype)
    print(f"[tile] case {case} index_dtype={index_dtype} rows={b.num_rows}", flush=True)
    d = H.upload(b)
    H.run_metadata(d)
    scores = H.run_scores(d)
    check_scores(b, scores, list(range(b.num_rows)))


def test_tile_equals_unit_scorer_bitwise(gpu_lib):
    """Rows of one 300-row request (tile kernel) against the same rows as 300
    one-row requests on the same pages (unit kernel, launched alone since the
    batch has at most 64 rows per call)."""
    b = syn.make_batch("tileu", 710, [6000], [300], topk=8, num_q_heads=16)
    d = H.upload(b)
    H.run_metadata(d)
    big = H.run_scores(d)
    # the same rows in calls of 50 one-row requests: request i has length
    # 6000 - 300 + i + 1 and the first request's block table
    ld_s = b.ld_s
    got = np.empty_like(big)
    for c0 in range(0, 300, 50):
        n = 50
        seq = torch.tensor([6000 - 300 + c0 + i + 1 for i in range(n)], dtype=torch.int32, device="cuda")
        qls = torch.ones(n, dtype=torch.int32, device="cuda")
        bt = d.block_table.repeat(n, 1).contiguous()
        meta = [torch.empty(n + 1, dtype=torch.int32, device="cuda") for _ in range(4)] + \
               [torch.empty(n, dtype=torch.int32, device="cuda") for _ in range(2)]
        cb = msa.make_batch(seq, qls, bt, *meta, n, n, 6000, b.num_pages)
        msa.msa_build_metadata(cb)
        sc = torch.full((n, ld_s), 7.0, dtype=torch.float32, device="cuda")
        iq = d.index_q[c0:c0 + n].contiguous()
        msa.msa_index_score(cb, iq, d.index_k, sc, ld_s)
        got[c0:c0 + n] = sc.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), big.view(np.uint32))

"""msa_sparse_decode_static — the fused step with its workspace in the
library's fixed device array (for callers that cannot allocate) — against
msa_sparse_decode_ex given a caller workspace of the same size: on calls in a
row, the second with a smaller batch, then a prefill-sized batch whose
block-major workspace fits the array (so both take the block-major path),
then the first batch again (the array keeps the previous call's bytes), every
output is bitwise equal.
"""
import numpy as np
import pytest
import torch

import block_sparse_paged_msa_amd as msa
import msa_synth as syn
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _decode(d, static, with_scores):
    b = d.host
    N, hq = b.num_rows, b.num_q_heads
    o = H.alloc_decode(d)
    lse = torch.full((N, hq), 7.0, dtype=torch.float32, device="cuda")
    scores = o.scores if with_scores else None
    if static:
        msa.msa_sparse_decode_static(d.cbatch, d.index_q, d.index_k, d.index_scale, d.q, hq, d.ckv, b.topk,
                                     b.sm_scale, None, o.out, lse, o.table, o.ctx, o.sel, scores, b.ld_s)
    else:
        ws = torch.full((msa.MSA_STATIC_SCRATCH_BYTES,), 0x3F, dtype=torch.uint8, device="cuda")
        msa.msa_sparse_decode_ex(d.cbatch, d.index_q, d.index_k, d.index_scale, d.q, hq, d.ckv, b.topk,
                                 b.sm_scale, None, o.out, lse, o.table, o.ctx, o.sel, scores, b.ld_s, ws,
                                 msa.MSA_STATIC_SCRATCH_BYTES)
    torch.cuda.synchronize()
    return [t.cpu() for t in (o.out, lse, o.table, o.ctx, o.sel)] + ([o.scores.cpu()] if with_scores else [])


def test_static_scratch_decode_matches_caller_workspace(gpu_lib):
    big = syn.config("fp8_kv", scale_mode=syn.SCALE_PER_TOKEN_HEAD)
    small = syn.make_batch("static2", 901, [9000, 700, 129], [1, 2, 1], topk=16, num_q_heads=16)
    prefill = syn.make_batch("static3", 902, [6000, 5000, 300], [2100, 1, 1], topk=2, num_q_heads=16)
    db, ds, dp = H.upload(big), H.upload(small), H.upload(prefill)
    need_big = msa.msa_workspace_bytes(big.num_rows, 16, 128 * big.topk, big.ld_s)
    assert 0 < need_big <= msa.MSA_STATIC_SCRATCH_BYTES
    need_bm = msa.msa_decode_workspace_bytes(prefill.num_rows, prefill.max_seq_len, 16, prefill.topk, prefill.ld_s)
    need_rows = msa.msa_workspace_bytes(prefill.num_rows, 16, 128 * prefill.topk, prefill.ld_s)
    assert need_rows < need_bm <= msa.MSA_STATIC_SCRATCH_BYTES  # the block-major path is taken
    print(f"[static] rows {big.num_rows}, {small.num_rows}, {prefill.num_rows} (block-major); "
          f"scratch need {need_big} / {need_bm} B", flush=True)
    # scores in the scratch (no caller score buffer), then a caller score buffer
    for name, d, with_scores in (("big", db, False), ("small", ds, True), ("block-major", dp, False),
                                 ("big again", db, False)):
        got = _decode(d, True, with_scores)
        want = _decode(d, False, with_scores)
        for i, (g, w) in enumerate(zip(got, want)):
            assert torch.equal(g, w), f"{name}: output {i} differs"
        assert np.isfinite(H.bf16_to_np(got[0].cuda())).all()
        print(f"[static] {name}: bitwise equal", flush=True)

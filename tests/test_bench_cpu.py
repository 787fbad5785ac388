"""Host logic of bench.py, on the CPU: the refusal of more than one GPU, the
number of cache copies cycled (at least 768 MB of touched bytes between two
uses of one copy, three times the 256 MB Infinity Cache), and the algorithmic
byte count of a step, worked out by hand for the one-row workload."""
import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import msa_synth as syn  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1",
                        "--warmup", "0"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stdout + r.stderr


@pytest.mark.parametrize("idx_fp8", [False, True])
@pytest.mark.parametrize("total_len", [2048, 50_000, 196_608, 262_144, 896_611, 3_000_000, 40_000_000])
def test_cache_copies_keep_768_mb_between_reuses(total_len, idx_fp8):
    # the score launch touches every visible index key once: 256 B a token
    # (bf16) or 132 B (e4m3fn codes and a 4-byte scale)
    b = types.SimpleNamespace(seq_lens=np.array([total_len // 2, total_len - total_len // 2], dtype=np.int32))
    per_copy = total_len * (132 if idx_fp8 else 256)
    c = bench.copies_for(b, idx_fp8)
    assert 2 <= c <= bench.MAX_COPIES
    if c < bench.MAX_COPIES:
        assert (c - 1) * per_copy >= 768e6          # enough
        assert c == 2 or (c - 2) * per_copy < 768e6  # and no more than needed


def test_algorithmic_bytes_of_the_one_row_step():
    # one request of 2048 tokens, one query row, 8 query heads, top-k 4,
    # bf16 K/V with no scales, 16 score columns; the row attends 512 tokens
    b = syn.config("tiny")
    assert (b.num_rows, b.num_q_heads, b.ld_s, b.topk, b.num_reqs) == (1, 8, 16, 4, 1)
    index_k = 2048 * 128 * 2              # every visible index key once
    index_q = 128 * 2
    kv = 512 * (128 * 2 + 128 * 2)        # K and V rows of the attended tokens
    q_out = 8 * 128 * 2 * 2               # queries read, outputs written
    scores = 16 * 4 * 2                   # written by the scorer, read by the selection
    table, ctx, sel = 8 * 4 * 4, 4, 4 * 4
    metadata = 6 * 4 + 2 * 4              # six per-request entries, row_req and row_pos
    got = bench.algorithmic_bytes(b, [512])
    assert got["step"] == index_k + index_q + kv + q_out + scores + table + ctx + sel + metadata
    assert got["score"] == index_k + index_q + 16 * 4
    assert got["kv"] == kv


def test_per_token_head_scales_add_eight_bytes_a_token():
    b = types.SimpleNamespace(num_rows=2, num_q_heads=16, ld_s=8, topk=2, kv_dtype=1, scale_mode=2,
                              seq_lens=np.array([1000], dtype=np.int32), index_scale=np.ones(1), num_reqs=1)
    got = bench.algorithmic_bytes(b, [200, 56])
    # fp8 K and V rows (128 B each) and one fp32 scale each per token
    assert got["kv"] == 256 * (2 * 128 + 2 * 4)
    # an fp8 index key: 128 codes and its 4-byte scale
    assert got["score"] == 1000 * 132 + 2 * 256 + 2 * 8 * 4

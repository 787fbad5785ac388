"""The C ABI library loads, exports what include/msa.h declares, and rejects
bad arguments on the host without launching anything (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_paged_msa_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:msa_status|size_t|const char\*|int32_t)\s+(msa_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return msa.load()


def test_header_declares_the_path_entry_points():
    names = header_functions()
    for want in ("msa_build_metadata", "msa_index_score", "msa_topk_block_table",
                 "msa_sparse_paged_attn", "msa_sparse_decode", "msa_index_score_ex",
                 "msa_sparse_paged_attn_ex", "msa_sparse_decode_ex", "msa_cache_insert",
                 "msa_cache_insert_ex", "msa_workspace_bytes", "msa_decode_workspace_bytes"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", msa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (msa_\w+)", out))
    assert exported == set(header_functions())
    assert set(msa.EXPORTS) == exported


def test_library_makes_no_host_round_trips():
    # no copy, synchronisation or allocation call is imported by the library
    out = subprocess.run(["nm", "-D", "--undefined-only", msa.LIB_PATH], capture_output=True, text=True).stdout
    for bad in ("hipMemcpy", "Synchronize", "hipMalloc", "hipFree", "hipMemset", "hipHostRegister"):
        assert bad not in out, bad


def test_status_strings(lib):
    assert msa.status_string(0) == "MSA_OK"
    assert msa.status_string(-3) == "MSA_ERR_WORKSPACE"
    assert msa.msa_version() >= 100


def test_workspace_bytes_monotone_and_aligned():
    a = msa.msa_workspace_bytes(8, 16, 2048, 0)
    b = msa.msa_workspace_bytes(8, 16, 2048, 256)
    c = msa.msa_workspace_bytes(16, 16, 2048, 256)
    assert 0 < a < b <= c
    assert a % 256 == 0 and b % 256 == 0
    assert msa.msa_workspace_bytes(-1, 16, 1, 0) == 0


def test_decode_workspace_bytes_block_major_layout():
    # below 2048 rows the fused step's per-row workspace; from 2048 rows the
    # block-major one: per row and head group, topk slots of 32 fp32 (m, l)
    # and 16x128 fp16, plus one 8-byte selection word per 32 blocks, 64 KiB
    # of per-block row counts, each region rounded up to 256 bytes, then the
    # scores when ld_s > 0
    def up(x):
        return (x + 255) // 256 * 256
    assert msa.msa_decode_workspace_bytes(100, 32768, 16, 32, 0) == msa.msa_workspace_bytes(100, 16, 128 * 32, 0)
    n, L, hq, topk, ld_s = 8198, 32768, 16, 32, 256
    slots = up(n * 1 * topk * (32 * 4 + 16 * 128 * 2))
    words = up(n * ((L // 128 + 31) // 32) * 8)
    counts = 16384 * 4
    got = msa.msa_decode_workspace_bytes(n, L, hq, topk, 0)
    assert got == max(slots + words + counts, msa.msa_workspace_bytes(n, hq, 128 * topk, 0))
    with_scores = msa.msa_decode_workspace_bytes(n, L, hq, topk, ld_s)
    assert with_scores == max(slots + words + counts + up(n * ld_s * 4),
                              msa.msa_workspace_bytes(n, hq, 128 * topk, ld_s))
    # two head groups double the slots
    assert msa.msa_decode_workspace_bytes(n, L, 24, topk, 0) >= 2 * slots
    for bad in ((-1, L, hq, topk, 0), (n, -1, hq, topk, 0), (n, L, 0, topk, 0), (n, L, hq, 0, 0), (n, L, hq, topk, -1)):
        assert msa.msa_decode_workspace_bytes(*bad) == 0


@pytest.fixture(autouse=True)
def _no_gpu_for_fake_pointers(request):
    # these tests pass made-up device addresses that validation must reject; on
    # a machine with a GPU a validation bug would launch on them, so they only
    # run where no GPU is visible
    if request.node.name.startswith(("test_metadata_rejects", "test_index_score", "test_topk_rejects",
                                     "test_attention_rejects", "test_empty_calls", "test_decode_rejects",
                                     "test_insert_rejects", "test_ex_entry_points")):
        import torch
        if torch.cuda.is_available():
            pytest.skip("fake device pointers are only passed where no GPU is visible")


def _fake_batch(**kw):
    base = dict(seq_lens=0x1000, query_lens=0x2000, block_table=0x3000, cu_seqlens_q=0x4000,
                cu_seqlens_k=0x5000, cu_blocks=0x6000, cu_units=0x7000, row_req=0x8000, row_pos=0x9000,
                num_reqs=2, num_rows=2, ld_bt=4, max_seq_len=512, num_pages=8)
    base.update(kw)
    return msa.MsaBatch(**base)


def _fake_kv(**kw):
    base = dict(k_cache=0x1000, v_cache=0x2000, k_scale=0, v_scale=0, kv_dtype=0, scale_mode=0,
                num_kv_heads=1, num_pages=8)
    base.update(kw)
    return msa.MsaKV(**base)


def _code(fn, *args):
    try:
        fn(*args)
    except msa.MsaError as e:
        return e.status
    return 0


# Each of these must fail host-side validation before any launch.
@pytest.mark.parametrize("batch,expect", [
    (dict(num_reqs=-1), msa.MSA_ERR_INVALID_ARG),
    (dict(num_reqs=9000), msa.MSA_ERR_UNSUPPORTED),
    (dict(max_seq_len=(1 << 20) + 1), msa.MSA_ERR_UNSUPPORTED),
    (dict(seq_lens=0), msa.MSA_ERR_INVALID_ARG),
    (dict(cu_units=0), msa.MSA_ERR_INVALID_ARG),
    (dict(ld_bt=0), msa.MSA_ERR_INVALID_ARG),
    (dict(num_reqs=0, num_rows=3), msa.MSA_ERR_INVALID_ARG),
    (dict(num_pages=(1 << 24) + 1), msa.MSA_ERR_UNSUPPORTED),
])
def test_metadata_rejects(batch, expect):
    assert _code(msa.msa_build_metadata, _fake_batch(**batch), 0) == expect


def test_index_score_rejects_small_ld_s():
    assert _code(msa.msa_index_score, _fake_batch(), 0x1, 0x2, 0x3, 3, 0) == msa.MSA_ERR_UNSUPPORTED
    assert _code(msa.msa_index_score, _fake_batch(), 0, 0x2, 0x3, 4, 0) == msa.MSA_ERR_INVALID_ARG


def test_topk_rejects():
    b = _fake_batch()
    assert _code(msa.msa_topk_block_table, b, 0x1, 4, 0, 0x2, 0x3, None, 0) == msa.MSA_ERR_INVALID_ARG
    assert _code(msa.msa_topk_block_table, b, 0x1, 4, 9000, 0x2, 0x3, None, 0) == msa.MSA_ERR_UNSUPPORTED
    assert _code(msa.msa_topk_block_table, b, 0x1, 2, 4, 0x2, 0x3, None, 0) == msa.MSA_ERR_UNSUPPORTED
    assert _code(msa.msa_topk_block_table, b, 0x1, 4, 4, 0, 0x3, None, 0) == msa.MSA_ERR_INVALID_ARG


@pytest.mark.parametrize("kv,expect", [
    (dict(num_kv_heads=2), msa.MSA_ERR_UNSUPPORTED),
    (dict(kv_dtype=1, scale_mode=0), msa.MSA_ERR_UNSUPPORTED),
    (dict(kv_dtype=1, scale_mode=2, k_scale=0x10, v_scale=0), msa.MSA_ERR_INVALID_ARG),
    (dict(kv_dtype=5), msa.MSA_ERR_INVALID_ARG),
    (dict(k_cache=0), msa.MSA_ERR_INVALID_ARG),
    (dict(num_pages=(1 << 24) + 1), msa.MSA_ERR_UNSUPPORTED),
])
def test_attention_rejects_kv(kv, expect):
    assert _code(msa.msa_sparse_paged_attn, 0x1, 4, 16, _fake_kv(**kv), 0x2, 8, 0x3, 128, 0.1,
                 0x4, 0x5, 1 << 20, 0) == expect


def test_attention_rejects_heads_table_and_workspace():
    kv = _fake_kv()
    assert _code(msa.msa_sparse_paged_attn, 0x1, 4, 200, kv, 0x2, 8, 0x3, 128, 0.1, 0x4, 0x5, 1 << 20, 0) \
        == msa.MSA_ERR_UNSUPPORTED
    assert _code(msa.msa_sparse_paged_attn, 0x1, 4, 16, kv, 0x2, 7, 0x3, 128, 0.1, 0x4, 0x5, 1 << 20, 0) \
        == msa.MSA_ERR_INVALID_ARG
    # a grid past 2^31 workgroups (2^22 rows x 8 head groups x 128 splits of
    # 2^20 tokens) is refused, not truncated
    assert _code(msa.msa_sparse_paged_attn, 0x1, 1 << 22, 128, kv, 0x2, 1 << 16, 0x3, 1 << 20, 0.1, 0x4, 0x5,
                 1 << 62, 0) == msa.MSA_ERR_UNSUPPORTED
    # no row attends more tokens than a request can hold
    assert _code(msa.msa_sparse_paged_attn, 0x1, 4, 16, kv, 0x2, 1 << 20, 0x3, (1 << 20) + 1, 0.1, 0x4, 0x5,
                 1 << 40, 0) == msa.MSA_ERR_UNSUPPORTED
    # 4 rows of 4096 tokens are split over several workgroups: partials need space
    need = msa.msa_workspace_bytes(4, 16, 4096, 0)
    assert need > 0
    assert _code(msa.msa_sparse_paged_attn, 0x1, 4, 16, kv, 0x2, 256, 0x3, 4096, 0.1, 0x4, 0x5, need - 1, 0) \
        == msa.MSA_ERR_WORKSPACE
    assert _code(msa.msa_sparse_paged_attn, 0x1, 4, 16, kv, 0x2, 256, 0x3, 4096, 0.1, 0x4, 0, need, 0) \
        == msa.MSA_ERR_WORKSPACE


def test_empty_calls_are_noops():
    kv = _fake_kv()
    assert _code(msa.msa_sparse_paged_attn, 0x1, 0, 16, kv, 0x2, 8, 0x3, 128, 0.1, 0x4, 0, 0, 0) == 0
    b = _fake_batch(num_reqs=0, num_rows=0)
    assert _code(msa.msa_build_metadata, b, 0) == 0
    assert _code(msa.msa_index_score, b, 0x1, 0x2, 0x3, 4, 0) == 0


def test_decode_rejects_before_launch():
    b = _fake_batch()
    kv = _fake_kv()
    args = [b, 0x1, 0x2, 0x3, 16, kv, 4, 0.1, 0x4, 0x5, 0x6, None, None, 4, 0x7, 1 << 30, 0]
    bad = list(args)
    bad[6] = 0                              # topk
    assert _code(msa.msa_sparse_decode, *bad) == msa.MSA_ERR_INVALID_ARG
    bad = list(args)
    bad[13] = 2                             # ld_s below ceil(512/128)
    assert _code(msa.msa_sparse_decode, *bad) == msa.MSA_ERR_UNSUPPORTED
    bad = list(args)
    bad[15] = 16                            # workspace too small
    assert _code(msa.msa_sparse_decode, *bad) == msa.MSA_ERR_WORKSPACE
    bad = list(args)
    bad[5] = _fake_kv(num_pages=9)          # caches and batch disagree on P
    assert _code(msa.msa_sparse_decode, *bad) == msa.MSA_ERR_INVALID_ARG


def test_ex_entry_points_check_like_the_plain_ones():
    kv = _fake_kv()
    # attention: heads, table stride, workspace, empty call
    assert _code(msa.msa_sparse_paged_attn_ex, 0x1, 4, 200, kv, 0x2, 8, 0x3, 128, 0.1, 0x9, 0x4, 0xA, 0x5,
                 1 << 20, 0) == msa.MSA_ERR_UNSUPPORTED
    assert _code(msa.msa_sparse_paged_attn_ex, 0x1, 4, 16, kv, 0x2, 7, 0x3, 128, 0.1, 0x9, 0x4, 0xA, 0x5,
                 1 << 20, 0) == msa.MSA_ERR_INVALID_ARG
    need = msa.msa_workspace_bytes(4, 16, 4096, 0)
    assert _code(msa.msa_sparse_paged_attn_ex, 0x1, 4, 16, kv, 0x2, 256, 0x3, 4096, 0.1, 0x9, 0x4, 0xA, 0x5,
                 need - 1, 0) == msa.MSA_ERR_WORKSPACE
    assert _code(msa.msa_sparse_paged_attn_ex, 0x1, 0, 16, kv, 0x2, 8, 0x3, 128, 0.1, 0x9, 0x4, 0xA, 0, 0,
                 0) == 0
    # decode: top-k, ld_s, workspace
    b = _fake_batch()
    args = [b, 0x1, 0x2, 0xB, 0x3, 16, kv, 4, 0.1, 0x9, 0x4, 0xA, 0x5, 0x6, None, None, 4, 0x7, 1 << 30, 0]
    for idx, val, expect in ((7, 0, msa.MSA_ERR_INVALID_ARG), (16, 2, msa.MSA_ERR_UNSUPPORTED),
                             (18, 16, msa.MSA_ERR_WORKSPACE)):
        bad = list(args)
        bad[idx] = val
        assert _code(msa.msa_sparse_decode_ex, *bad) == expect
    # index scores: ld_s too small; insert: index rows with no index cache
    assert _code(msa.msa_index_score_ex, b, 0x1, 0x2, 0xB, 0x3, 2, 0) == msa.MSA_ERR_UNSUPPORTED
    assert _code(msa.msa_cache_insert_ex, 4, 0x1, 0x2, 0x3, kv, 0x4, 0, 0xB, 0) == msa.MSA_ERR_INVALID_ARG


def test_decode_rejects_static_scratch_overflow():
    """msa_sparse_decode_static checks like msa_sparse_decode_ex and refuses a
    launch whose workspace would not fit its fixed 32 MiB array, before any
    device call."""
    kv = _fake_kv()
    b = _fake_batch()
    args = [b, 0x1, 0x2, None, 0x3, 16, kv, 4, 0.1, None, 0x4, None, 0x5, 0x6, None, 0x8, 4, 0]
    for idx, val, expect in ((7, 0, msa.MSA_ERR_INVALID_ARG), (16, 2, msa.MSA_ERR_UNSUPPORTED),
                             (5, 200, msa.MSA_ERR_UNSUPPORTED)):
        bad = list(args)
        bad[idx] = val
        assert _code(msa.msa_sparse_decode_static, *bad) == expect
    # 4096 rows whose scores would live in the workspace: 4096 x 8192 x 4 B > 32 MiB
    big = _fake_batch(num_rows=4096, max_seq_len=1 << 20, ld_bt=8192)
    need = msa.msa_workspace_bytes(4096, 16, 128 * 4, 8192)
    assert need > msa.MSA_STATIC_SCRATCH_BYTES
    bad = list(args)
    bad[0], bad[15], bad[16] = big, None, 8192
    assert _code(msa.msa_sparse_decode_static, *bad) == msa.MSA_ERR_WORKSPACE


@pytest.mark.parametrize("args,kv,expect", [
    (dict(num_tokens=-1), {}, msa.MSA_ERR_INVALID_ARG),
    (dict(slot_mapping=0), {}, msa.MSA_ERR_INVALID_ARG),
    (dict(k_new=0), {}, msa.MSA_ERR_INVALID_ARG),
    (dict(v_new=0), {}, msa.MSA_ERR_INVALID_ARG),
    (dict(index_k=0), {}, msa.MSA_ERR_INVALID_ARG),     # index rows given, no index cache
    ({}, dict(num_kv_heads=2), msa.MSA_ERR_UNSUPPORTED),
    ({}, dict(kv_dtype=1, scale_mode=0), msa.MSA_ERR_UNSUPPORTED),
    ({}, dict(kv_dtype=1, scale_mode=1, k_scale=0x10, v_scale=0), msa.MSA_ERR_INVALID_ARG),
    (dict(num_tokens=0), {}, 0),                          # nothing to do: no launch
])
def test_insert_rejects(args, kv, expect):
    a = dict(num_tokens=4, slot_mapping=0x1, k_new=0x2, v_new=0x3, index_k_new=0x4, index_k=0x5)
    a.update(args)
    assert _code(msa.msa_cache_insert, a["num_tokens"], a["slot_mapping"], a["k_new"], a["v_new"],
                 _fake_kv(**kv), a["index_k_new"], a["index_k"], 0) == expect


def test_insert_rejects_more_pages_than_slots_name():
    # slots are int32 128*page + offset: caches past 2^24 pages are refused
    kv = _fake_kv(num_pages=(1 << 24) + 1)
    assert _code(msa.msa_cache_insert, 4, 0x1, 0x2, 0x3, kv, None, None, 0) == msa.MSA_ERR_UNSUPPORTED
    assert msa.MSA_MAX_PAGES == 1 << 24

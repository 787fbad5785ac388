"""Caches of more than 4 GiB a plane: a batch's pages moved on the device to
ids whose byte offsets lie past 2^32 in the index-K, K and V planes give the
same results, bit for bit, as at their original ids (no result depends on
where a page lives; a wrapped 32-bit offset would read or write another page),
for the per-row path (fp8 K/V, bf16 or fp8 index), the block-major path and
the cache insert. Only the pages a batch uses are written in the large
caches; the rest is never read."""
import dataclasses

import numpy as np
import pytest
import torch

import block_sparse_paged_msa_amd as msa
import msa_synth as syn
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _grow(t, per_page, off, P):
    big = torch.empty((per_page * (off + P),) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
    big[per_page * off:] = t
    return big


def _relocate(d, off):
    """The same batch with every page id raised by `off` (caches of off + P
    pages, the block table shifted)."""
    b = d.host
    P = b.num_pages
    r = dataclasses.replace(d)
    r.index_k = _grow(d.index_k, 1, off, P)
    r.k_cache, r.v_cache = _grow(d.k_cache, 8, off, P), _grow(d.v_cache, 8, off, P)
    if b.scale_mode == syn.SCALE_PER_TOKEN_HEAD:
        r.k_scale, r.v_scale = _grow(d.k_scale, 8, off, P), _grow(d.v_scale, 8, off, P)
    if d.index_scale is not None:
        r.index_scale = _grow(d.index_scale, 1, off, P)
    r.block_table = d.block_table + off
    r.cbatch = msa.make_batch(r.seq_lens, r.query_lens, r.block_table, r.cu_q, r.cu_k, r.cu_blocks, r.cu_units,
                              r.row_req, r.row_pos, b.num_reqs, b.num_rows, b.max_seq_len, off + P)
    r.ckv = msa.make_kv(r.k_cache, r.v_cache, b.kv_dtype, b.scale_mode, off + P, r.k_scale, r.v_scale)
    return r


def _decode(d, block_major):
    b = d.host
    o = H.alloc_decode(d)
    if block_major:
        wsb = msa.msa_decode_workspace_bytes(b.num_rows, b.max_seq_len, b.num_q_heads, b.topk, 0)
        o.ws, o.wsb = torch.empty((wsb,), dtype=torch.uint8, device="cuda"), wsb
    H.run_decode(d, o)
    torch.cuda.synchronize()
    return o


CASES = [
    # (name, lengths, query rows, top-k, kv dtype, scale mode, index dtype, page offset, block-major)
    ("fp8kv", [20000, 9000, 300], [1, 2, 1], 16, syn.KV_FP8, syn.SCALE_PER_TOKEN_HEAD, syn.INDEX_BF16, 300000, False),
    ("fp8index", [20000, 9000, 300], [1, 2, 1], 16, syn.KV_FP8, syn.SCALE_PER_TOKEN_HEAD, syn.INDEX_FP8, 300000,
     False),
    ("blockmajor", [6000, 3000], [2100, 1], 8, syn.KV_BF16, syn.SCALE_NONE, syn.INDEX_BF16, 140000, True),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_decode_on_pages_past_4gib(gpu_lib, case):
    name, L, ql, topk, kv, sm, idx, off, bm = CASES[case]
    b = syn.make_batch("large_" + name, 950 + case, L, ql, topk=topk, num_q_heads=16, kv_dtype=kv, scale_mode=sm,
                       index_dtype=idx)
    elt = 2 if kv == syn.KV_BF16 else 1
    assert off * 128 * 128 * 2 // (2 if idx == syn.INDEX_FP8 else 1) > 2 ** 32   # index-K offsets
    assert 8 * off * 16 * 128 * elt > 2 ** 32                                     # K and V offsets
    print(f"[large] {name}: rows={b.num_rows} pages {off}..{off + b.num_pages}", flush=True)
    d = H.upload(b)
    ref = _decode(d, bm)
    far = _decode(_relocate(d, off), bm)
    for field in ("out", "ctx", "sel", "scores"):
        assert torch.equal(getattr(far, field), getattr(ref, field)), field
    # the page-16 table names the moved sub-pages: 8*off more on the kept columns
    sel = ref.sel.cpu().numpy()
    kept = (sel >= 0).sum(axis=1)
    cols = np.arange(8 * topk)[None, :] < 8 * kept[:, None]
    want = np.where(cols, ref.table.cpu().numpy().astype(np.int64) + 8 * off, 0)
    assert np.array_equal(far.table.cpu().numpy(), want)
    assert np.isfinite(H.bf16_to_np(far.out)).all()


@pytest.mark.parametrize("layout", ["in_order", "scattered"])
def test_insert_on_pages_past_4gib(gpu_lib, layout):
    """256 new tokens into two pages at ids 0 and 1, and into the same pages
    moved to ids 300000 and 300001 of large fp8 caches (per-token-head scales,
    bf16 index): the two pages hold the same bytes afterwards."""
    off, P, T = 300000, 2, 256
    g = torch.Generator(device="cpu").manual_seed(960)
    k_new = (torch.randn((T, 1, 128), generator=g) * 2).to(torch.bfloat16).view(torch.int16).cuda()
    v_new = (torch.randn((T, 1, 128), generator=g) * 2).to(torch.bfloat16).view(torch.int16).cuda()
    i_new = torch.randn((T, 128), generator=g).to(torch.bfloat16).view(torch.int16).cuda()
    t = torch.arange(T)
    slots = t if layout == "in_order" else torch.randperm(P * 128, generator=g)[:T]
    slots = slots.to(torch.int32)
    print(f"[large] insert {layout}: pages {off}, {off + 1}", flush=True)

    def caches(pages):
        kc = torch.zeros((8 * pages, 1, 2048), dtype=torch.uint8, device="cuda")
        vc = torch.zeros((8 * pages, 1, 2048), dtype=torch.uint8, device="cuda")
        ks = torch.ones((8 * pages, 16, 1), dtype=torch.float32, device="cuda")
        vs = torch.ones((8 * pages, 16, 1), dtype=torch.float32, device="cuda")
        ik = torch.zeros((pages, 128 * 128), dtype=torch.int16, device="cuda")
        return kc, vc, ks, vs, ik

    near = caches(P)
    kv = msa.make_kv(near[0], near[1], syn.KV_FP8, syn.SCALE_PER_TOKEN_HEAD, P, near[2], near[3])
    msa.msa_cache_insert(T, slots.cuda(), k_new, v_new, kv, i_new, near[4])
    far = [torch.empty((8 * (off + P),) + tuple(x.shape[1:]), dtype=x.dtype, device="cuda") for x in near[:4]]
    far.append(torch.empty((off + P, 128 * 128), dtype=torch.int16, device="cuda"))
    for x in far[:4]:
        x[8 * off:] = 0 if x.dtype == torch.uint8 else 1.0
    far[4][off:] = 0
    kv_far = msa.make_kv(far[0], far[1], syn.KV_FP8, syn.SCALE_PER_TOKEN_HEAD, off + P, far[2], far[3])
    msa.msa_cache_insert(T, (slots + 128 * off).cuda(), k_new, v_new, kv_far, i_new, far[4])
    torch.cuda.synchronize()
    for a, b_, per in zip(near, far, (8, 8, 8, 8, 1)):
        assert torch.equal(b_[per * off:], a)

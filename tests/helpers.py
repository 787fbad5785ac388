"""Test helpers: move a synthetic batch to the GPU and drive the C ABI through
the Python binding. Nothing here computes any step of the method."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import block_sparse_paged_msa_amd as msa
import msa_synth as syn

GUARD = 256          # sentinel elements on each side of every output buffer
SENTINEL_I32 = -0x5A5A5A5B
SENTINEL_F32 = 1.2345e30
SENTINEL_U16 = 0x7E55


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a.copy()).to(device)


def guarded(n: int, dtype: torch.dtype, fill, device="cuda"):
    """Buffer of n elements between two guard bands of sentinels; returns
    (full, view)."""
    full = torch.full((n + 2 * GUARD,), fill, dtype=dtype, device=device)
    return full, full[GUARD:GUARD + n]


def guards_intact(full: torch.Tensor, fill) -> bool:
    g = torch.cat([full[:GUARD], full[-GUARD:]])
    return bool((g == fill).all().item())


@dataclasses.dataclass
class DeviceBatch:
    host: syn.Batch
    seq_lens: torch.Tensor
    query_lens: torch.Tensor
    block_table: torch.Tensor
    cu_q: torch.Tensor
    cu_k: torch.Tensor
    cu_blocks: torch.Tensor
    cu_units: torch.Tensor
    row_req: torch.Tensor
    row_pos: torch.Tensor
    index_q: torch.Tensor
    index_k: torch.Tensor
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    k_scale: torch.Tensor | None
    v_scale: torch.Tensor | None
    cbatch: msa.MsaBatch = None
    ckv: msa.MsaKV = None
    index_scale: torch.Tensor | None = None   # set for an fp8 index cache


def upload(b: syn.Batch, device="cuda") -> DeviceBatch:
    R, N = b.num_reqs, b.num_rows
    i32 = dict(dtype=torch.int32, device=device)
    d = DeviceBatch(
        host=b,
        seq_lens=dev(b.seq_lens, device), query_lens=dev(b.query_lens, device),
        block_table=dev(b.block_table, device),
        cu_q=torch.full((R + 1,), -7, **i32), cu_k=torch.full((R + 1,), -7, **i32),
        cu_blocks=torch.full((R + 1,), -7, **i32), cu_units=torch.full((R + 1,), -7, **i32),
        row_req=torch.full((max(N, 1),), -7, **i32), row_pos=torch.full((max(N, 1),), -7, **i32),
        index_q=dev(b.index_q, device), index_k=dev(b.index_k, device), q=dev(b.q, device),
        k_cache=dev(b.k_cache, device), v_cache=dev(b.v_cache, device),
        k_scale=None if b.k_scale is None else dev(b.k_scale, device),
        v_scale=None if b.v_scale is None else dev(b.v_scale, device),
    )
    d.cbatch = msa.make_batch(d.seq_lens, d.query_lens, d.block_table, d.cu_q, d.cu_k, d.cu_blocks,
                              d.cu_units, d.row_req, d.row_pos, R, N, b.max_seq_len, b.num_pages)
    d.ckv = msa.make_kv(d.k_cache, d.v_cache, b.kv_dtype, b.scale_mode, b.num_pages, d.k_scale, d.v_scale)
    if b.index_scale is not None:
        d.index_scale = dev(b.index_scale, device)
    return d


def read_metadata(d: DeviceBatch) -> dict:
    """The batch metadata arrays as they are on the device (no launch)."""
    N = d.host.num_rows
    return {"cu_seqlens_q": d.cu_q.cpu().numpy(), "cu_seqlens_k": d.cu_k.cpu().numpy(),
            "cu_blocks": d.cu_blocks.cpu().numpy(), "cu_units": d.cu_units.cpu().numpy(),
            "row_req": d.row_req[:N].cpu().numpy(), "row_pos": d.row_pos[:N].cpu().numpy()}


def run_metadata(d: DeviceBatch) -> dict:
    msa.msa_build_metadata(d.cbatch)
    N = d.host.num_rows
    return {"cu_seqlens_q": d.cu_q.cpu().numpy(), "cu_seqlens_k": d.cu_k.cpu().numpy(),
            "cu_blocks": d.cu_blocks.cpu().numpy(), "cu_units": d.cu_units.cpu().numpy(),
            "row_req": d.row_req[:N].cpu().numpy(), "row_pos": d.row_pos[:N].cpu().numpy()}


def run_scores(d: DeviceBatch) -> np.ndarray:
    b = d.host
    full, scores = guarded(b.num_rows * b.ld_s, torch.float32, SENTINEL_F32)
    if d.index_scale is None:
        msa.msa_index_score(d.cbatch, d.index_q, d.index_k, scores, b.ld_s)
    else:
        msa.msa_index_score_ex(d.cbatch, d.index_q, d.index_k, d.index_scale, scores, b.ld_s)
    assert guards_intact(full, SENTINEL_F32), "index score wrote outside its buffer"
    return scores.view(b.num_rows, b.ld_s).cpu().numpy()


def run_topk(d: DeviceBatch, scores_np: np.ndarray, topk: int | None = None):
    b = d.host
    topk = b.topk if topk is None else topk
    s = torch.from_numpy(np.ascontiguousarray(scores_np, dtype=np.float32)).cuda()
    tfull, table = guarded(b.num_rows * 8 * topk, torch.int32, SENTINEL_I32)
    cfull, ctx = guarded(b.num_rows, torch.int32, SENTINEL_I32)
    sfull, sel = guarded(b.num_rows * topk, torch.int32, SENTINEL_I32)
    msa.msa_topk_block_table(d.cbatch, s, b.ld_s, topk, table, ctx, sel)
    for full in (tfull, cfull, sfull):
        assert guards_intact(full, SENTINEL_I32), "top-k wrote outside its buffers"
    return (table.view(b.num_rows, 8 * topk).cpu().numpy(), ctx.cpu().numpy(),
            sel.view(b.num_rows, topk).cpu().numpy())


def run_attn(d: DeviceBatch, table: np.ndarray, ctx: np.ndarray, max_ctx: int | None = None,
             sm_scale: float | None = None) -> np.ndarray:
    b = d.host
    N, hq = b.num_rows, b.num_q_heads
    ld_table = table.shape[1]
    max_ctx = 16 * ld_table if max_ctx is None else max_ctx
    sm_scale = b.sm_scale if sm_scale is None else sm_scale
    t = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).cuda()
    c = torch.from_numpy(np.ascontiguousarray(ctx, dtype=np.int32)).cuda()
    ofull, out = guarded(N * hq * 128, torch.int16, SENTINEL_U16)
    wsb = msa.msa_workspace_bytes(N, hq, max_ctx, 0)
    ws = torch.full((wsb // 4 + 1,), 0x3F3F3F3F, dtype=torch.int32, device="cuda")  # garbage on entry
    msa.msa_sparse_paged_attn(d.q, N, hq, d.ckv, t, ld_table, c, max_ctx, sm_scale, out, ws, wsb)
    assert guards_intact(ofull, SENTINEL_U16), "attention wrote outside its output"
    return bf16_to_np(out.view(N, hq, 128))


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.bfloat16).float().cpu().numpy().astype(np.float64)


@dataclasses.dataclass
class DecodeOut:
    out: torch.Tensor
    table: torch.Tensor
    ctx: torch.Tensor
    sel: torch.Tensor
    scores: torch.Tensor
    ws: torch.Tensor
    wsb: int


def alloc_decode(d: DeviceBatch, with_scores: bool = True) -> DecodeOut:
    b = d.host
    N, hq, topk = b.num_rows, b.num_q_heads, b.topk
    wsb = msa.msa_workspace_bytes(N, hq, 128 * topk, 0 if with_scores else b.ld_s)
    return DecodeOut(
        out=torch.full((N, hq, 128), 0x7FC0, dtype=torch.int16, device="cuda"),  # bf16 NaN: unwritten shows
        table=torch.full((N, 8 * topk), SENTINEL_I32, dtype=torch.int32, device="cuda"),
        ctx=torch.full((N,), SENTINEL_I32, dtype=torch.int32, device="cuda"),
        sel=torch.full((N, topk), SENTINEL_I32, dtype=torch.int32, device="cuda"),
        scores=torch.zeros((N, b.ld_s), dtype=torch.float32, device="cuda"),
        ws=torch.full((wsb // 4 + 1,), 0x3F3F3F3F, dtype=torch.int32, device="cuda"),
        wsb=wsb)


def run_decode(d: DeviceBatch, o: DecodeOut, with_scores: bool = True) -> None:
    b = d.host
    if d.index_scale is None:
        msa.msa_sparse_decode(d.cbatch, d.index_q, d.index_k, d.q, b.num_q_heads, d.ckv, b.topk, b.sm_scale,
                              o.out, o.table, o.ctx, o.sel, o.scores if with_scores else None, b.ld_s, o.ws, o.wsb)
    else:
        msa.msa_sparse_decode_ex(d.cbatch, d.index_q, d.index_k, d.index_scale, d.q, b.num_q_heads, d.ckv, b.topk,
                                 b.sm_scale, None, o.out, None, o.table, o.ctx, o.sel,
                                 o.scores if with_scores else None, b.ld_s, o.ws, o.wsb)


def run_attn_lse(d: DeviceBatch, table: np.ndarray, ctx: np.ndarray, sinks: np.ndarray | None,
                 max_ctx: int | None = None):
    """msa_sparse_paged_attn_ex on a given table; returns (out, lse)."""
    b = d.host
    N, hq = b.num_rows, b.num_q_heads
    ld_table = table.shape[1]
    max_ctx = 16 * ld_table if max_ctx is None else max_ctx
    t = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).cuda()
    c = torch.from_numpy(np.ascontiguousarray(ctx, dtype=np.int32)).cuda()
    s = None if sinks is None else torch.from_numpy(np.ascontiguousarray(sinks, dtype=np.float32)).cuda()
    ofull, out = guarded(N * hq * 128, torch.int16, SENTINEL_U16)
    lfull, lse = guarded(N * hq, torch.float32, SENTINEL_F32)
    wsb = msa.msa_workspace_bytes(N, hq, max_ctx, 0)
    ws = torch.full((wsb // 4 + 1,), 0x3F3F3F3F, dtype=torch.int32, device="cuda")
    msa.msa_sparse_paged_attn_ex(d.q, N, hq, d.ckv, t, ld_table, c, max_ctx, b.sm_scale, s, out, lse, ws, wsb)
    assert guards_intact(ofull, SENTINEL_U16), "attention wrote outside its output"
    assert guards_intact(lfull, SENTINEL_F32), "attention wrote outside its lse"
    return bf16_to_np(out.view(N, hq, 128)), lse.view(N, hq).cpu().numpy().astype(np.float64)


def run_decode_lse(d: DeviceBatch, o: DecodeOut, sinks: np.ndarray | None) -> np.ndarray:
    """msa_sparse_decode_ex into o (with the batch's index cache); returns the lse [N][Hq]."""
    b = d.host
    s = None if sinks is None else torch.from_numpy(np.ascontiguousarray(sinks, dtype=np.float32)).cuda()
    lfull, lse = guarded(b.num_rows * b.num_q_heads, torch.float32, SENTINEL_F32)
    msa.msa_sparse_decode_ex(d.cbatch, d.index_q, d.index_k, d.index_scale, d.q, b.num_q_heads, d.ckv, b.topk,
                             b.sm_scale, s, o.out, lse, o.table, o.ctx, o.sel, o.scores, b.ld_s, o.ws, o.wsb)
    assert guards_intact(lfull, SENTINEL_F32), "decode wrote outside its lse"
    return lse.view(b.num_rows, b.num_q_heads).cpu().numpy().astype(np.float64)


def plant_nan_tails(b: syn.Batch) -> int:
    """Write NaN into every cache slot past each request's last token (the
    rest of its last page): index keys (and their fp8 scales), K, V and
    per-token-head K/V scales. Those slots are never visible, so no output may
    change; returns the number of slots planted."""
    bf16_nan, fp8_nan = np.uint16(0x7FC0), np.uint8(0x7F)
    planted = 0
    for r in range(b.num_reqs):
        L = int(b.seq_lens[r])
        if L % 128 == 0:
            continue
        page = int(b.block_table[r, (L - 1) // 128])
        for t in range(L % 128, 128):
            sub, ts = 8 * page + t // 16, t % 16
            if b.index_scale is None:
                b.index_k[page, t // 16, :, :, ts, :] = bf16_nan
            else:
                b.index_k[page, t // 16, :, :, ts, :] = fp8_nan
                b.index_scale.reshape(-1)[page * 128 + t] = np.float32(np.nan)
            nan = bf16_nan if b.kv_dtype == syn.KV_BF16 else fp8_nan
            b.k_cache[sub, :, :, :, ts, :] = nan
            b.v_cache[sub, :, :, ts] = nan
            if b.scale_mode == syn.SCALE_PER_TOKEN_HEAD:
                b.k_scale[sub, ts, :] = np.float32(np.nan)
                b.v_scale[sub, ts, :] = np.float32(np.nan)
            planted += 1
    return planted

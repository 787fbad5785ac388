"""Python binding of the block-sparse paged decode-attention library (libmsa.so).

Argument marshalling only: each function takes torch device tensors (or raw
device addresses), builds the C structs of ``include/msa.h`` and calls the entry
point of the same name on torch's current HIP stream. Every step of the path
runs in the library's HIP kernels; there is no Python or CPU fallback, and a
missing library raises.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmsa.so")

MSA_OK = 0
MSA_ERR_INVALID_ARG = -1
MSA_ERR_UNSUPPORTED = -2
MSA_ERR_WORKSPACE = -3
MSA_ERR_HIP = -4

MSA_KV_BF16 = 0
MSA_KV_FP8_E4M3FN = 1
MSA_SCALE_NONE = 0
MSA_SCALE_SCALAR = 1
MSA_SCALE_PER_TOKEN_HEAD = 2
MSA_STATIC_SCRATCH_BYTES = 32 << 20   # workspace inside the library used by msa_sparse_decode_static
MSA_MAX_PAGES = 1 << 24               # physical pages a batch or cache may name

EXPORTS = (
    "msa_build_metadata", "msa_index_score", "msa_topk_block_table", "msa_sparse_paged_attn",
    "msa_sparse_decode", "msa_index_score_ex", "msa_sparse_paged_attn_ex", "msa_sparse_decode_ex",
    "msa_sparse_decode_static", "msa_cache_insert", "msa_cache_insert_ex",
    "msa_workspace_bytes", "msa_decode_workspace_bytes", "msa_status_string", "msa_version",
)


class MsaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


class MsaBatch(ctypes.Structure):
    _fields_ = [
        ("seq_lens", ctypes.c_void_p), ("query_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p), ("cu_blocks", ctypes.c_void_p),
        ("cu_units", ctypes.c_void_p), ("row_req", ctypes.c_void_p), ("row_pos", ctypes.c_void_p),
        ("num_reqs", ctypes.c_int32), ("num_rows", ctypes.c_int32), ("ld_bt", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32), ("num_pages", ctypes.c_int32),
    ]


class MsaKV(ctypes.Structure):
    _fields_ = [
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("kv_dtype", ctypes.c_int32), ("scale_mode", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("num_pages", ctypes.c_int32),
    ]


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libmsa.so (raises if it is missing: the path has no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m block_sparse_paged_msa_amd.build`")
    # torch carries its own HIP runtime under the same soname: load torch
    # first so that the library binds to that runtime instead of bringing in
    # a second one (kernels of one runtime are invalid in the other)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    bp, kp = ctypes.POINTER(MsaBatch), ctypes.POINTER(MsaKV)
    sig = {
        "msa_build_metadata": ([vp, bp], i32),
        "msa_index_score": ([vp, bp, vp, vp, vp, i32], i32),
        "msa_topk_block_table": ([vp, bp, vp, i32, i32, vp, vp, vp], i32),
        "msa_sparse_paged_attn": ([vp, vp, i32, i32, kp, vp, i32, vp, i32, f32, vp, vp, sz], i32),
        "msa_sparse_decode": ([vp, bp, vp, vp, vp, i32, kp, i32, f32, vp, vp, vp, vp, vp, i32, vp, sz], i32),
        "msa_index_score_ex": ([vp, bp, vp, vp, vp, vp, i32], i32),
        "msa_sparse_paged_attn_ex": ([vp, vp, i32, i32, kp, vp, i32, vp, i32, f32, vp, vp, vp, vp, sz], i32),
        "msa_sparse_decode_ex": ([vp, bp, vp, vp, vp, vp, i32, kp, i32, f32, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                  sz], i32),
        "msa_sparse_decode_static": ([vp, bp, vp, vp, vp, vp, i32, kp, i32, f32, vp, vp, vp, vp, vp, vp, vp,
                                      i32], i32),
        "msa_cache_insert": ([vp, i32, vp, vp, vp, kp, vp, vp], i32),
        "msa_cache_insert_ex": ([vp, i32, vp, vp, vp, kp, vp, vp, vp], i32),
        "msa_workspace_bytes": ([i32, i32, i32, i32], sz),
        "msa_decode_workspace_bytes": ([i32, i32, i32, i32, i32], sz),
        "msa_status_string": ([i32], ctypes.c_char_p),
        "msa_version": ([], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().msa_status_string(status).decode()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, st: int) -> None:
    if st != MSA_OK:
        raise MsaError(fn, st)


def make_batch(seq_lens, query_lens, block_table, cu_seqlens_q, cu_seqlens_k, cu_blocks, cu_units,
               row_req, row_pos, num_reqs: int, num_rows: int, max_seq_len: int, num_pages: int,
               ld_bt: int | None = None) -> MsaBatch:
    """C struct for a batch whose arrays are device tensors (int32)."""
    return MsaBatch(_ptr(seq_lens), _ptr(query_lens), _ptr(block_table), _ptr(cu_seqlens_q),
                    _ptr(cu_seqlens_k), _ptr(cu_blocks), _ptr(cu_units), _ptr(row_req), _ptr(row_pos),
                    num_reqs, num_rows, block_table.shape[1] if ld_bt is None else ld_bt,
                    max_seq_len, num_pages)


def make_kv(k_cache, v_cache, kv_dtype: int, scale_mode: int, num_pages: int, k_scale=None, v_scale=None,
            num_kv_heads: int = 1) -> MsaKV:
    return MsaKV(_ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), kv_dtype, scale_mode,
                 num_kv_heads, num_pages)


def msa_build_metadata(batch: MsaBatch, stream=None) -> None:
    _check("msa_build_metadata", load().msa_build_metadata(_stream(stream), ctypes.byref(batch)))


def msa_index_score(batch: MsaBatch, index_q, index_k, block_scores, ld_s: int, stream=None) -> None:
    _check("msa_index_score", load().msa_index_score(
        _stream(stream), ctypes.byref(batch), _ptr(index_q), _ptr(index_k), _ptr(block_scores), ld_s))


def msa_topk_block_table(batch: MsaBatch, block_scores, ld_s: int, topk: int, sparse_table, ctx_lens,
                         sel_blocks=None, stream=None) -> None:
    _check("msa_topk_block_table", load().msa_topk_block_table(
        _stream(stream), ctypes.byref(batch), _ptr(block_scores), ld_s, topk, _ptr(sparse_table),
        _ptr(ctx_lens), _ptr(sel_blocks)))


def msa_sparse_paged_attn(q, num_rows: int, num_q_heads: int, kv: MsaKV, sparse_table, ld_table: int,
                          ctx_lens, max_ctx: int, sm_scale: float, out, workspace, workspace_bytes: int,
                          stream=None) -> None:
    _check("msa_sparse_paged_attn", load().msa_sparse_paged_attn(
        _stream(stream), _ptr(q), num_rows, num_q_heads, ctypes.byref(kv), _ptr(sparse_table), ld_table,
        _ptr(ctx_lens), max_ctx, sm_scale, _ptr(out), _ptr(workspace), workspace_bytes))


def msa_sparse_decode(batch: MsaBatch, index_q, index_k, q, num_q_heads: int, kv: MsaKV, topk: int,
                      sm_scale: float, out, sparse_table, ctx_lens, sel_blocks, block_scores, ld_s: int,
                      workspace, workspace_bytes: int, stream=None) -> None:
    _check("msa_sparse_decode", load().msa_sparse_decode(
        _stream(stream), ctypes.byref(batch), _ptr(index_q), _ptr(index_k), _ptr(q), num_q_heads,
        ctypes.byref(kv), topk, sm_scale, _ptr(out), _ptr(sparse_table), _ptr(ctx_lens), _ptr(sel_blocks),
        _ptr(block_scores), ld_s, _ptr(workspace), workspace_bytes))


def msa_index_score_ex(batch: MsaBatch, index_q, index_k, index_k_scale, block_scores, ld_s: int,
                       stream=None) -> None:
    _check("msa_index_score_ex", load().msa_index_score_ex(
        _stream(stream), ctypes.byref(batch), _ptr(index_q), _ptr(index_k), _ptr(index_k_scale),
        _ptr(block_scores), ld_s))


def msa_sparse_paged_attn_ex(q, num_rows: int, num_q_heads: int, kv: MsaKV, sparse_table, ld_table: int,
                             ctx_lens, max_ctx: int, sm_scale: float, sinks, out, lse, workspace,
                             workspace_bytes: int, stream=None) -> None:
    _check("msa_sparse_paged_attn_ex", load().msa_sparse_paged_attn_ex(
        _stream(stream), _ptr(q), num_rows, num_q_heads, ctypes.byref(kv), _ptr(sparse_table), ld_table,
        _ptr(ctx_lens), max_ctx, sm_scale, _ptr(sinks), _ptr(out), _ptr(lse), _ptr(workspace), workspace_bytes))


def msa_sparse_decode_ex(batch: MsaBatch, index_q, index_k, index_k_scale, q, num_q_heads: int, kv: MsaKV,
                         topk: int, sm_scale: float, sinks, out, lse, sparse_table, ctx_lens, sel_blocks,
                         block_scores, ld_s: int, workspace, workspace_bytes: int, stream=None) -> None:
    _check("msa_sparse_decode_ex", load().msa_sparse_decode_ex(
        _stream(stream), ctypes.byref(batch), _ptr(index_q), _ptr(index_k), _ptr(index_k_scale), _ptr(q),
        num_q_heads, ctypes.byref(kv), topk, sm_scale, _ptr(sinks), _ptr(out), _ptr(lse), _ptr(sparse_table),
        _ptr(ctx_lens), _ptr(sel_blocks), _ptr(block_scores), ld_s, _ptr(workspace), workspace_bytes))


def msa_sparse_decode_static(batch: MsaBatch, index_q, index_k, index_k_scale, q, num_q_heads: int, kv: MsaKV,
                             topk: int, sm_scale: float, sinks, out, lse, sparse_table, ctx_lens, sel_blocks,
                             block_scores, ld_s: int, stream=None) -> None:
    _check("msa_sparse_decode_static", load().msa_sparse_decode_static(
        _stream(stream), ctypes.byref(batch), _ptr(index_q), _ptr(index_k), _ptr(index_k_scale), _ptr(q),
        num_q_heads, ctypes.byref(kv), topk, sm_scale, _ptr(sinks), _ptr(out), _ptr(lse), _ptr(sparse_table),
        _ptr(ctx_lens), _ptr(sel_blocks), _ptr(block_scores), ld_s))


def msa_cache_insert(num_tokens: int, slot_mapping, k_new, v_new, kv: MsaKV, index_k_new, index_k,
                     stream=None) -> None:
    _check("msa_cache_insert", load().msa_cache_insert(
        _stream(stream), num_tokens, _ptr(slot_mapping), _ptr(k_new), _ptr(v_new), ctypes.byref(kv),
        _ptr(index_k_new), _ptr(index_k)))


def msa_cache_insert_ex(num_tokens: int, slot_mapping, k_new, v_new, kv: MsaKV, index_k_new, index_k,
                        index_k_scale, stream=None) -> None:
    _check("msa_cache_insert_ex", load().msa_cache_insert_ex(
        _stream(stream), num_tokens, _ptr(slot_mapping), _ptr(k_new), _ptr(v_new), ctypes.byref(kv),
        _ptr(index_k_new), _ptr(index_k), _ptr(index_k_scale)))


def msa_workspace_bytes(num_rows: int, num_q_heads: int, max_ctx: int, ld_s: int) -> int:
    return int(load().msa_workspace_bytes(num_rows, num_q_heads, max_ctx, ld_s))


def msa_decode_workspace_bytes(num_rows: int, max_seq_len: int, num_q_heads: int, topk: int, ld_s: int) -> int:
    return int(load().msa_decode_workspace_bytes(num_rows, max_seq_len, num_q_heads, topk, ld_s))


def msa_version() -> int:
    return int(load().msa_version())

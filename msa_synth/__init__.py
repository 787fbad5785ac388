"""Seeded synthetic inputs for block-sparse paged decode attention.

This module only draws random numbers and places them into the buffer layouts
that the library's header documents. It holds none of the method's arithmetic
(no scoring, pooling, selection, table expansion, dequantisation or softmax), so
the CPU oracle and the GPU path can both consume its arrays without sharing any
code of the method.

Generator
---------
* ``splitmix64`` (Steele, Lea, Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): state advances by the golden gamma
  ``0x9E3779B97F4A7C15``; output mixing uses the published constants
  ``0xBF58476D1CE4E5B9`` / ``0x94D049BB133111EB`` with shifts 30/27/31.
* uniform doubles take the top 53 bits; normals come from Box-Muller using both
  the cosine and the sine branch.
* bf16 values are ``bf16(fp32(x))`` with round-to-nearest-even at each step.
* fp8 e4m3fn codes are produced by torch's ``float8_e4m3fn`` cast (RNE) of the
  fp32 value; N(0,1) draws never approach the 448 limit.

Draw order per batch: lengths, page permutation, index_q, index_k, q, k, v,
scales, index-K scales (fp8 index caches only). Everything is a pure function
of ``(config, seed)``; an fp8 index cache draws the same normals as a bf16 one,
so every other array is the same in both.

Buffer layouts (see ``include/msa.h``)
--------------------------------------
A 16-token tile of 128-dim rows is stored "MFMA-shuffled" as [4][4][16][8]:
(32-dim chunk, 8-dim group, token, element); dim d of a token is at chunk d//32,
group (d%32)//8, element d%8.
* ``index_k``  [P][8][4][4][16][8] bf16 bits (uint16): page, 16-token tile, shuffled tile;
  or e4m3fn codes (uint8) in the same order, with ``index_scale`` [P][128] fp32
  (one scale per token slot of each page).
* ``k_cache``  [P*8][Hkv][4][4][16][8]: sub-page, KV head, shuffled tile.
* ``v_cache``  [P*8][Hkv][128][16]: dim-major inside each 16-token sub-page.
* per-token-head scales [P*8][16][Hkv] fp32; scalar scales are a [1] array.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

GOLDEN_GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

PAGE = 128      # tokens per physical KV / index-K page
SUB = 16        # tokens per sub-page of the page-16 view
HEAD_DIM = 128
INDEX_DIM = 128

TILE_SHAPE = (4, 4, SUB, 8)                 # shuffled 16-token x 128-dim tile
INDEX_PAGE_SHAPE = (PAGE // SUB,) + TILE_SHAPE

KV_BF16 = 0
KV_FP8 = 1
SCALE_NONE = 0
SCALE_SCALAR = 1
SCALE_PER_TOKEN_HEAD = 2
INDEX_BF16 = 0
INDEX_FP8 = 1


class SplitMix64:
    """Vectorised splitmix64 stream."""

    def __init__(self, seed: int):
        self.state = int(seed) & MASK64

    def next_u64(self, n: int) -> np.ndarray:
        n = int(n)
        if n == 0:
            return np.zeros(0, dtype=np.uint64)
        i = np.arange(1, n + 1, dtype=np.uint64)
        z = np.uint64(self.state) + i * np.uint64(GOLDEN_GAMMA)
        self.state = (self.state + n * GOLDEN_GAMMA) & MASK64
        z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX2)
        return z ^ (z >> np.uint64(31))

    def uniform(self, n: int) -> np.ndarray:
        """Doubles in [0, 1)."""
        return (self.next_u64(n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)

    def uniform_open0(self, n: int) -> np.ndarray:
        """Doubles in (0, 1]."""
        return ((self.next_u64(n) >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)

    def integers(self, lo: int, hi: int, n: int) -> np.ndarray:
        """Integers uniform on the inclusive range [lo, hi]."""
        span = hi - lo + 1
        v = lo + np.floor(self.uniform(n) * span).astype(np.int64)
        return np.minimum(v, hi)

    def normal(self, n: int) -> np.ndarray:
        """N(0,1) draws by Box-Muller, chunked to bound memory."""
        out = np.empty(n, dtype=np.float64)
        chunk = 1 << 22
        pos = 0
        while pos < n:
            m = min(chunk, n - pos)
            pairs = (m + 1) // 2
            u1 = self.uniform_open0(pairs)
            u2 = self.uniform(pairs)
            r = np.sqrt(-2.0 * np.log(u1))
            th = 2.0 * math.pi * u2
            z = np.empty(2 * pairs, dtype=np.float64)
            z[0::2] = r * np.cos(th)
            z[1::2] = r * np.sin(th)
            out[pos:pos + m] = z[:m]
            pos += m
        return out

    def permutation(self, n: int) -> np.ndarray:
        keys = self.next_u64(n)
        return np.argsort(keys, kind="stable").astype(np.int32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16(fp32(x)) bit patterns, round-to-nearest-even at both steps."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def to_e4m3fn_codes(x: np.ndarray) -> np.ndarray:
    """OCP fp8 e4m3fn codes of fp32(x), via torch's RNE cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def bf16_normal(rng: SplitMix64, shape) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    chunk = 1 << 24
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        out[s:s + m] = to_bf16_bits(rng.normal(m))
    return out.reshape(shape)


def fp8_normal(rng: SplitMix64, shape) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    chunk = 1 << 24
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        out[s:s + m] = to_e4m3fn_codes(rng.normal(m))
    return out.reshape(shape)


@dataclasses.dataclass
class Batch:
    """One batch of synthetic inputs, all host numpy arrays."""
    name: str
    seed: int
    seq_lens: np.ndarray        # [R] int32
    query_lens: np.ndarray      # [R] int32
    block_table: np.ndarray     # [R][ld_bt] int32 physical page-128 ids
    num_pages: int
    max_seq_len: int            # host upper bound used to size ld_S and grids
    topk: int
    num_q_heads: int
    num_kv_heads: int
    kv_dtype: int
    scale_mode: int
    sm_scale: float
    index_q: np.ndarray         # [N][128] uint16 (bf16 bits)
    index_k: np.ndarray         # [P][8][4][4][16][8] uint16
    q: np.ndarray               # [N][Hq][128] uint16
    k_cache: np.ndarray         # [8P][Hkv][4][4][16][8] uint16 or uint8
    v_cache: np.ndarray         # [8P][Hkv][128][16] uint16 or uint8
    k_scale: np.ndarray | None  # [1] or [8P][16][Hkv] float32
    v_scale: np.ndarray | None
    index_dtype: int = INDEX_BF16
    index_scale: np.ndarray | None = None   # [P][128] float32 (fp8 index only)

    @property
    def num_reqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_rows(self) -> int:
        return int(self.query_lens.sum())

    @property
    def ld_bt(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def ld_s(self) -> int:
        return max(1, -(-self.max_seq_len // PAGE))


def make_batch(name: str, seed: int, seq_lens, query_lens, topk: int, num_q_heads: int,
               *, kv_dtype: int = KV_BF16, scale_mode: int = SCALE_NONE,
               permute_pages: bool = True, max_seq_len: int | None = None,
               scale_lo: float = 0.5, scale_hi: float = 2.0, num_kv_heads: int = 1,
               extra_pages: int = 0, ld_bt: int | None = None, data: bool = True,
               index_dtype: int = INDEX_BF16) -> Batch:
    """Build a batch from explicit lengths (lengths are not drawn here).
    With ``data=False`` only lengths and the block table are drawn; the tensor
    fields are empty (for tests of metadata and selection alone)."""
    rng = SplitMix64(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    query_lens = np.asarray(query_lens, dtype=np.int32)
    return _fill(rng, name, seed, seq_lens, query_lens, topk, num_q_heads, kv_dtype,
                 scale_mode, permute_pages, max_seq_len, scale_lo, scale_hi,
                 num_kv_heads, extra_pages, ld_bt, data, index_dtype)


def _fill(rng, name, seed, seq_lens, query_lens, topk, hq, kv_dtype, scale_mode,
          permute_pages, max_seq_len, scale_lo, scale_hi, hkv, extra_pages, ld_bt, data=True,
          index_dtype=INDEX_BF16):
    R = int(seq_lens.shape[0])
    nblk = [-(-int(L) // PAGE) for L in seq_lens]
    P = int(sum(nblk)) + int(extra_pages)
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max()) if R else 0
    if ld_bt is None:
        ld_bt = max(1, max(nblk) if R else 1)
    perm = rng.permutation(P) if permute_pages else np.arange(P, dtype=np.int32)
    bt = np.zeros((R, ld_bt), dtype=np.int32)
    pos = 0
    for r in range(R):
        bt[r, :nblk[r]] = perm[pos:pos + nblk[r]]
        pos += nblk[r]
    N = int(query_lens.sum())
    if not data:
        e16, e8 = np.zeros(0, np.uint16), np.zeros(0, np.uint8)
        return Batch(name=name, seed=seed, seq_lens=seq_lens, query_lens=query_lens,
                     block_table=bt, num_pages=P, max_seq_len=int(max_seq_len), topk=int(topk),
                     num_q_heads=int(hq), num_kv_heads=int(hkv), kv_dtype=int(kv_dtype),
                     scale_mode=int(scale_mode), sm_scale=1.0 / math.sqrt(HEAD_DIM),
                     index_q=e16, index_k=e16, q=e16,
                     k_cache=e16 if kv_dtype == KV_BF16 else e8,
                     v_cache=e16 if kv_dtype == KV_BF16 else e8, k_scale=None, v_scale=None)
    index_q = bf16_normal(rng, (N, INDEX_DIM))
    if index_dtype == INDEX_FP8:
        index_k = fp8_normal(rng, (P,) + INDEX_PAGE_SHAPE)
    else:
        index_k = bf16_normal(rng, (P,) + INDEX_PAGE_SHAPE)
    q = bf16_normal(rng, (N, hq, HEAD_DIM))
    if kv_dtype == KV_BF16:
        k_cache = bf16_normal(rng, (P * 8, hkv) + TILE_SHAPE)
        v_cache = bf16_normal(rng, (P * 8, hkv, HEAD_DIM, SUB))
    else:
        k_cache = fp8_normal(rng, (P * 8, hkv) + TILE_SHAPE)
        v_cache = fp8_normal(rng, (P * 8, hkv, HEAD_DIM, SUB))
    k_scale = v_scale = None
    if scale_mode == SCALE_SCALAR:
        k_scale = (scale_lo + (scale_hi - scale_lo) * rng.uniform(1)).astype(np.float32)
        v_scale = (scale_lo + (scale_hi - scale_lo) * rng.uniform(1)).astype(np.float32)
    elif scale_mode == SCALE_PER_TOKEN_HEAD:
        n = P * 8 * SUB * hkv
        k_scale = (scale_lo + (scale_hi - scale_lo) * rng.uniform(n)).astype(np.float32).reshape(P * 8, SUB, hkv)
        v_scale = (scale_lo + (scale_hi - scale_lo) * rng.uniform(n)).astype(np.float32).reshape(P * 8, SUB, hkv)
    index_scale = None
    if index_dtype == INDEX_FP8:
        index_scale = (scale_lo + (scale_hi - scale_lo) * rng.uniform(P * PAGE)).astype(np.float32) \
            .reshape(P, PAGE)
    return Batch(name=name, seed=seed, seq_lens=seq_lens, query_lens=query_lens,
                 block_table=bt, num_pages=P, max_seq_len=int(max_seq_len), topk=int(topk),
                 num_q_heads=int(hq), num_kv_heads=int(hkv), kv_dtype=int(kv_dtype),
                 scale_mode=int(scale_mode), sm_scale=1.0 / math.sqrt(HEAD_DIM),
                 index_q=index_q, index_k=index_k, q=q, k_cache=k_cache, v_cache=v_cache,
                 k_scale=k_scale, v_scale=v_scale, index_dtype=int(index_dtype), index_scale=index_scale)


# ---------------------------------------------------------------------------
# The five workloads. Lengths are the first draws of each seed's stream.
# ---------------------------------------------------------------------------
CONFIG_NAMES = ("tiny", "bf16_batch", "spec_decode", "fp8_kv", "mixed_prefill")


def config(name: str, *, scale_mode: int | None = None, index_dtype: int = INDEX_BF16) -> Batch:
    """The named workload with its fixed seed.

    tiny          1 request, 1 row, L=2048, identity pages, top-k 4, 8 q heads (seed 0)
    bf16_batch    8 requests x 1 row, L~U{8192..32768}, permuted pages, top-k 16 (seed 1)
    spec_decode   4 requests x 4 rows, L=65536, top-k 32 (seed 2)
    fp8_kv        11 requests x 1 row, L~U{32768..131072}, fp8 e4m3fn K/V with
                  per-token-head scales U[0.5,2] (or one scalar pair), top-k 64 (seed 3)
    mixed_prefill 6 decode rows at L=16384 then 2 prefill requests of 4096 rows on
                  28672 prior tokens (L=32768), top-k 32 (seed 4)
    ``index_dtype=INDEX_FP8`` gives any of them an fp8 index cache (codes from
    the same normals, per-token scales drawn last).
    """
    if name == "tiny":
        rng = SplitMix64(0)
        return _fill(rng, name, 0, np.array([2048], np.int32), np.array([1], np.int32), 4, 8,
                     KV_BF16, SCALE_NONE, False, 2048, 0.5, 2.0, 1, 0, None, index_dtype=index_dtype)
    if name == "bf16_batch":
        rng = SplitMix64(1)
        L = rng.integers(8192, 32768, 8).astype(np.int32)
        return _fill(rng, name, 1, L, np.ones(8, np.int32), 16, 16, KV_BF16, SCALE_NONE,
                     True, 32768, 0.5, 2.0, 1, 0, None, index_dtype=index_dtype)
    if name == "spec_decode":
        rng = SplitMix64(2)
        L = np.full(4, 65536, np.int32)
        return _fill(rng, name, 2, L, np.full(4, 4, np.int32), 32, 16, KV_BF16, SCALE_NONE,
                     True, 65536, 0.5, 2.0, 1, 0, None, index_dtype=index_dtype)
    if name == "fp8_kv":
        rng = SplitMix64(3)
        L = rng.integers(32768, 131072, 11).astype(np.int32)
        sm = SCALE_PER_TOKEN_HEAD if scale_mode is None else scale_mode
        return _fill(rng, name, 3, L, np.ones(11, np.int32), 64, 16, KV_FP8, sm,
                     True, 131072, 0.5, 2.0, 1, 0, None, index_dtype=index_dtype)
    if name == "mixed_prefill":
        rng = SplitMix64(4)
        L = np.array([16384] * 6 + [32768] * 2, np.int32)
        ql = np.array([1] * 6 + [4096] * 2, np.int32)
        return _fill(rng, name, 4, L, ql, 32, 16, KV_BF16, SCALE_NONE,
                     True, 32768, 0.5, 2.0, 1, 0, None, index_dtype=index_dtype)
    raise KeyError(name)


def random_batch(seed: int, num_reqs: int, max_len: int, *, max_q: int = 1, topk: int = 8,
                 num_q_heads: int = 16, kv_dtype: int = KV_BF16,
                 scale_mode: int = SCALE_NONE, min_len: int = 1) -> Batch:
    """Small random batch for parity tests: ragged lengths, mixed query lengths."""
    rng = SplitMix64(seed)
    L = rng.integers(min_len, max_len, num_reqs).astype(np.int32)
    ql = np.minimum(rng.integers(1, max_q, num_reqs), L).astype(np.int32) if max_q > 1 \
        else np.ones(num_reqs, np.int32)
    return _fill(rng, f"random{seed}", seed, L, ql, topk, num_q_heads, kv_dtype, scale_mode,
                 True, int(max_len), 0.5, 2.0, 1, 0, None)

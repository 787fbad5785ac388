"""CPU oracle for MiniMax-M3-style block-sparse paged decode attention.

TEST INFRASTRUCTURE ONLY. This module is the plain, slow reference that the HIP
library is checked against. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import it; the product path never does. It
shares no code with the HIP library: it reads host numpy arrays in the layouts
the C header documents and computes every step from its definition, in float64.

Sources (prhub.com.cn summaries of vLLM pull requests):
  [P1] PR #47287, "add ROCm AITER sparse paged attention for MiniMax-M3"
  [P2] PR #54682, "optimise gfx950 MiniMax-M3 decode index and top-k"
  [P3] PR #54404, "attention sinks for ROCm AITER sparse MLA, with a decode
       operator that returns natural-log LSE"
  [P4] PR #56170, "MiniMax M3 cu_seqlens_k first element zeroed on the device"
The FP8 index cache is named on the [P2] page (相关 PRs: #52664 routes FP8
decode scoring and top-k elsewhere, #53448 adds optional FP8 index storage);
its format is a reading (below).
Section names are the pages' own: 功能与动机 (motivation), 实现拆解 (implementation
breakdown, numbered items), 关键源码片段 (key source excerpt), 评论区精华 (review
highlights), 风险与影响 (risks).

Readings taken where the pages are silent:
  * index score = raw dot product of the row's index query with each token's
    index key, one index head, no scale;
  * pooling over a 128-token block = max over the block's visible tokens;
  * a row at absolute position pos sees keys 0..pos (v = pos + 1);
  * selection keeps min(topk, nb) blocks under the total order (score
    descending, block id ascending, -0 == +0) and lists them by ascending id;
  * every selected block expands to all 8 of its 16-token sub-pages, sub-page i
    of physical page P being 8P + i; the row is zero-filled up to 8*topk;
  * attention over the selected blocks' visible tokens with an exact softmax;
    FP8 values are dequantised as scale x e4m3fn(code);
  * an FP8 index cache holds e4m3fn codes with one fp32 scale per token
    (index key = scale x e4m3fn(code)); the index query stays bf16;
  * the log-sum-exp is that of the scaled logits over the attended tokens
    alone; a head's sink adds exp(sink) to its softmax denominator (a logit
    with no value vector) and leaves the log-sum-exp unchanged.

Parity status: every function here is pinned by tests/test_oracle_pins.py to
closed forms, brute force, library routines or invariants, except the modelling
readings above (score formula and pooling operator), which no page fixes:
that these match the real model is parity unpinned.
"""
from __future__ import annotations

import numpy as np

PAGE = 128       # tokens per KV / index-K page and per sparse block
SUB = 16         # tokens per sub-page of the page-16 view
SUBS_PER_PAGE = PAGE // SUB


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64: the bf16 pattern is the top half of
    an IEEE binary32 word."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit floating point E4M3 ("fn": finite, no infinities).

    Bit layout S.EEEE.MMM, exponent bias 7. E == 0 encodes subnormals
    (-1)^S * 2^-6 * M/8; otherwise (-1)^S * 2^(E-7) * (1 + M/8). The two codes
    S.1111.111 are NaN; S.1111.110 is the largest finite magnitude, 448.
    FP8 K/V are the storage format named in [P1] 实现拆解 item 2.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = sign * np.ldexp(m / 8.0, -6)
    val = np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, val)


# ---------------------------------------------------------------------------
# Step 1: batch metadata
# ---------------------------------------------------------------------------
def build_metadata(seq_lens: np.ndarray, query_lens: np.ndarray) -> dict:
    """Device-side batch metadata, [P4] 实现拆解 items 1-3 and 关键源码片段.

    cu_seqlens_k starts with a zero and continues with the running sum of the
    requests' KV lengths; cu_seqlens_q is the running start of each request's
    query rows; every query row gets its request id and absolute position,
    which is the request's prior context plus the row's offset inside the
    request's new tokens (context_len = seq_len - query_len). Decode rows come
    first and prefill rows after, so one formula covers both.
    cu_blocks counts the 128-token blocks of each request's KV.
    """
    L = [int(x) for x in seq_lens]
    ql = [int(x) for x in query_lens]
    R = len(L)
    cu_q = [0] * (R + 1)
    cu_k = [0] * (R + 1)
    cu_b = [0] * (R + 1)
    row_req, row_pos = [], []
    for r in range(R):
        cu_q[r + 1] = cu_q[r] + ql[r]
        cu_k[r + 1] = cu_k[r] + L[r]
        cu_b[r + 1] = cu_b[r] + (L[r] + PAGE - 1) // PAGE
        context_len = L[r] - ql[r]
        for i in range(ql[r]):
            row_req.append(r)
            row_pos.append(context_len + i)
    return {
        "cu_seqlens_q": np.array(cu_q, dtype=np.int64),
        "cu_seqlens_k": np.array(cu_k, dtype=np.int64),
        "cu_blocks": np.array(cu_b, dtype=np.int64),
        "row_req": np.array(row_req, dtype=np.int64),
        "row_pos": np.array(row_pos, dtype=np.int64),
    }


def visible_keys(row_pos: int) -> int:
    """A row at absolute position pos attends to keys 0..pos (causal)."""
    return int(row_pos) + 1


def num_blocks(v: int) -> int:
    return (int(v) + PAGE - 1) // PAGE


# ---------------------------------------------------------------------------
# Step 2: index scores and per-block pooling
# ---------------------------------------------------------------------------
def tile_row(tile: np.ndarray, tok: int) -> np.ndarray:
    """The 128 values of token `tok` of a stored 16-token tile. Tiles are kept
    as [4][4][16][8] (32-dim chunk, 8-dim group, token, element): dim d of the
    token is at [d // 32][(d % 32) // 8][tok][d % 8]."""
    return tile[:, :, tok, :].reshape(-1)


def index_keys_of_request(index_k_bits: np.ndarray, bt_row: np.ndarray, ntok: int,
                          index_scale: np.ndarray | None = None) -> np.ndarray:
    """Logical index keys [ntok][128] of one request: token t lives in physical
    page bt_row[t // 128], slot s = t % 128 (the page-128 cache, [P1] 实现拆解
    item 3), i.e. in 16-token tile s // 16 of the page, as token s % 16.
    With ``index_scale`` ([P][128] fp32) the pages hold e4m3fn codes and the
    key is index_scale[page][s] x e4m3fn(code) (the optional FP8 index cache
    of PR #53448, named on the [P2] page; per-token scale is a reading)."""
    out = np.empty((ntok, 128), dtype=np.float64)
    for j in range(num_blocks(ntok)):
        lo, hi = j * PAGE, min((j + 1) * PAGE, ntok)
        pid = int(bt_row[j])
        page = index_k_bits[pid]                          # [8][4][4][16][8]
        # (tile, chunk, group, token, element) -> (tile, token, chunk, group, element)
        rows = page.transpose(0, 3, 1, 2, 4).reshape(PAGE, 128)[: hi - lo]
        if index_scale is None:
            out[lo:hi] = bf16_to_f64(rows)
        else:
            sc = np.asarray(index_scale, dtype=np.float64)[pid, : hi - lo]
            out[lo:hi] = e4m3fn_to_f64(rows) * sc[:, None]
    return out


def token_scores(index_q_row: np.ndarray, keys: np.ndarray, v: int) -> np.ndarray:
    """Score of one query row against each visible token t < v: the dot product
    of the row's index query with the token's index key ([P2] 功能与动机 and
    实现拆解 item 1 name the per-row decode scorer; the formula is a reading)."""
    qi = bf16_to_f64(index_q_row)
    return keys[:v] @ qi


def pool_blocks(tok_scores: np.ndarray, nb: int) -> np.ndarray:
    """Block score = max of the token scores inside the 128-token block; the
    last block may be partial and pools over its visible tokens only."""
    out = np.empty(nb, dtype=np.float64)
    for b in range(nb):
        out[b] = np.max(tok_scores[b * PAGE:(b + 1) * PAGE])
    return out


def block_scores(index_q: np.ndarray, index_k: np.ndarray, block_table: np.ndarray,
                 seq_lens: np.ndarray, query_lens: np.ndarray, ld_s: int,
                 rows=None, index_scale: np.ndarray | None = None) -> np.ndarray:
    """[N][ld_s] pooled scores; -inf at and beyond each row's block count.

    ``rows`` restricts the computation to a subset of rows (others stay -inf);
    ``index_scale`` marks an FP8 index cache (see index_keys_of_request)."""
    meta = build_metadata(seq_lens, query_lens)
    N = len(meta["row_req"])
    out = np.full((N, ld_s), -np.inf, dtype=np.float64)
    want = range(N) if rows is None else sorted(set(int(r) for r in rows))
    by_req: dict[int, list[int]] = {}
    for n in want:
        by_req.setdefault(int(meta["row_req"][n]), []).append(n)
    for r, ns in by_req.items():
        keys = index_keys_of_request(index_k, block_table[r], int(seq_lens[r]), index_scale)
        for n in ns:
            v = visible_keys(meta["row_pos"][n])
            nb = num_blocks(v)
            out[n, :nb] = pool_blocks(token_scores(index_q[n], keys, v), nb)
    return out


# ---------------------------------------------------------------------------
# Step 3: top-k selection, page-16 table, context length
# ---------------------------------------------------------------------------
def select_blocks(scores_row: np.ndarray, nb: int, topk: int) -> np.ndarray:
    """Top-k blocks of one row ([P2] 实现拆解 item 1: the fused top-k picks each
    row's blocks): order the eligible blocks by score descending with the lower
    block id first among equals, keep the first min(topk, nb), and list them by
    ascending block id. Python float comparison treats -0.0 and +0.0 as equal."""
    cand = [(float(scores_row[b]), b) for b in range(nb)]
    ranked = sorted(cand, key=lambda sb: (-sb[0], sb[1]))   # stable
    keep = ranked[:min(topk, nb)]
    return np.array(sorted(b for _, b in keep), dtype=np.int64)


def select_blocks_by_rank(scores_row: np.ndarray, nb: int, topk: int) -> np.ndarray:
    """Second formulation of the same selection: block b is kept iff fewer than
    min(topk, nb) eligible blocks beat it (higher score, or equal score and
    lower id)."""
    kk = min(topk, nb)
    s = [float(scores_row[b]) for b in range(nb)]
    keep = []
    for b in range(nb):
        beaten_by = sum(1 for c in range(nb) if s[c] > s[b] or (s[c] == s[b] and c < b))
        if beaten_by < kk:
            keep.append(b)
    return np.array(keep, dtype=np.int64)


def sparse_table_row(sel: np.ndarray, bt_row: np.ndarray, topk: int) -> np.ndarray:
    """Page-16 sparse block table row ([P1] 实现拆解 item 3: a page-16 K/V view
    derived from the page-128 layout; [P2] 实现拆解 items 1 and 4: the table row
    is written from the selected values). Selected block j (in ascending order)
    occupies entries 8j..8j+7 = 8*bt_row[sel_j] + i; entries from 8*len(sel) up
    to the row width 8*topk are zero and nothing is written past the width
    ([P1] 评论区精华: the zero-padding store must stay inside the row)."""
    out = np.zeros(SUBS_PER_PAGE * topk, dtype=np.int64)
    for j, b in enumerate(sel):
        for i in range(SUBS_PER_PAGE):
            out[SUBS_PER_PAGE * j + i] = SUBS_PER_PAGE * int(bt_row[int(b)]) + i
    return out


def context_length(sel: np.ndarray, v: int) -> int:
    """Tokens the row attends to: each selected block contributes its visible
    tokens, min(128, v - 128*b) ([P2] 实现拆解 item 1: the fused pass also
    outputs context lengths)."""
    return int(sum(min(PAGE, int(v) - PAGE * int(b)) for b in sel))


def selection_row_outputs(sel: np.ndarray, topk: int) -> np.ndarray:
    """sel written as [topk] with -1 after the kept blocks."""
    out = np.full(topk, -1, dtype=np.int64)
    out[:len(sel)] = sel
    return out


# ---------------------------------------------------------------------------
# Step 4: sparse paged attention over the selected blocks
# ---------------------------------------------------------------------------
def kv_token(cache: np.ndarray, bt_row: np.ndarray, t: int, hkv: int, kv_dtype: int,
             plane: str) -> np.ndarray:
    """Raw stored values of one token for KV head hkv, addressed logically:
    physical page P = bt_row[t // 128], sub-page 8P + (t % 128) // 16, slot t % 16.
    K sub-pages are shuffled tiles [Hkv][4][4][16][8] (see tile_row); V
    sub-pages are dim-major [Hkv][128][16]."""
    page = int(bt_row[t // PAGE])
    sub = SUBS_PER_PAGE * page + (t % PAGE) // SUB
    slot = t % SUB
    raw = tile_row(cache[sub, hkv], slot) if plane == "k" else cache[sub, hkv, :, slot]
    return bf16_to_f64(raw) if kv_dtype == 0 else e4m3fn_to_f64(raw)


def token_scale(scale: np.ndarray | None, scale_mode: int, bt_row: np.ndarray, t: int,
                hkv: int) -> float:
    """FP8 K/V scale of one token ([P1] 实现拆解 item 2 and 关键文件: k_scale and
    v_scale, 'scalar' or 'per_token_head'). Per-token-head scales are stored
    [P][128][Hkv] (same as [8P][16][Hkv])."""
    if scale_mode == 0:
        return 1.0
    if scale_mode == 1:
        return float(np.asarray(scale).reshape(-1)[0])
    page = int(bt_row[t // PAGE])
    s = np.asarray(scale).reshape(-1, PAGE, np.asarray(scale).shape[-1])
    return float(s[page, t % PAGE, hkv])


def dequant_tokens(cache, scale, scale_mode, kv_dtype, bt_row, tokens, hkv, plane):
    """K-hat / V-hat rows: scale x stored value, float64."""
    out = np.empty((len(tokens), 128), dtype=np.float64)
    for i, t in enumerate(tokens):
        out[i] = token_scale(scale, scale_mode, bt_row, t, hkv) * \
            kv_token(cache, bt_row, t, hkv, kv_dtype, plane)
    return out


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float) -> np.ndarray:
    """Exact attention of query heads q [H][D] over keys k [T][D], values
    v [T][D]: two-pass softmax (max, then normalised exponentials)."""
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    z = sm_scale * (q @ k.T)                       # [H][T]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    return (e @ v) / e.sum(axis=1, keepdims=True)


def softmax_attention_lse(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float,
                          sinks: np.ndarray | None = None):
    """Attention of query heads q [H][D] over keys k [T][D], values v [T][D],
    with each head's natural-log log-sum-exp of its scaled logits
    z = sm_scale q k^T ([P3] 实现拆解 item 1: a decode operator that also
    returns natural-log LSE):  lse[h] = ln sum_t exp(z[h][t]).
    sinks [H] ([P3] 实现拆解 item 2: one float32 sink per head) add exp(sinks[h])
    to head h's softmax denominator; lse stays that of the keys alone.
    Returns (out [H][D], lse [H]); no keys give zeros and lse = -inf."""
    H = q.shape[0]
    if k.shape[0] == 0:
        return np.zeros((H, v.shape[1]), dtype=np.float64), np.full(H, -np.inf)
    z = sm_scale * (q @ k.T)                       # [H][T]
    m = z.max(axis=1)
    e = np.exp(z - m[:, None])
    den = e.sum(axis=1)
    lse = m + np.log(den)
    if sinks is not None:
        den = den + np.exp(np.asarray(sinks, dtype=np.float64) - m)
    return (e @ v) / den[:, None], lse


def sparse_attention_row(q_row_bits: np.ndarray, k_cache, v_cache, kv_dtype: int,
                         scale_mode: int, k_scale, v_scale, bt_row: np.ndarray,
                         sel: np.ndarray, v: int, sm_scale: float) -> np.ndarray:
    """Attention of one row's query heads over only the selected blocks' visible
    tokens ([P1] 功能与动机: attention over a small number of logical blocks;
    实现拆解 item 3: paged attention over the page-16 view). Tokens are walked
    logically through the request's page-128 table, not through the page-16
    table, so that the GPU's table walk is checked against the definition.
    Query head h reads KV head h // (Hq / Hkv)."""
    hq = q_row_bits.shape[0]
    hkv_n = k_cache.shape[1]
    group = hq // hkv_n
    tokens = [t for b in sel for t in range(PAGE * int(b), min(PAGE * (int(b) + 1), v))]
    q = bf16_to_f64(q_row_bits)
    out = np.zeros((hq, q.shape[1]), dtype=np.float64)
    for g in range(hkv_n):
        kh = dequant_tokens(k_cache, k_scale, scale_mode, kv_dtype, bt_row, tokens, g, "k")
        vh = dequant_tokens(v_cache, v_scale, scale_mode, kv_dtype, bt_row, tokens, g, "v")
        out[g * group:(g + 1) * group] = softmax_attention(q[g * group:(g + 1) * group], kh, vh, sm_scale)
    return out


def dense_causal_attention_row(q_row_bits, k_cache, v_cache, kv_dtype, scale_mode, k_scale,
                               v_scale, bt_row, v, sm_scale) -> np.ndarray:
    """Textbook causal attention of one row over every visible key t < v."""
    hq = q_row_bits.shape[0]
    hkv_n = k_cache.shape[1]
    group = hq // hkv_n
    q = bf16_to_f64(q_row_bits)
    out = np.zeros((hq, q.shape[1]), dtype=np.float64)
    tokens = list(range(int(v)))
    for g in range(hkv_n):
        kh = dequant_tokens(k_cache, k_scale, scale_mode, kv_dtype, bt_row, tokens, g, "k")
        vh = dequant_tokens(v_cache, v_scale, scale_mode, kv_dtype, bt_row, tokens, g, "v")
        for h in range(g * group, (g + 1) * group):
            z = np.array([sm_scale * float(q[h] @ kh[t]) for t in range(len(tokens))])
            if len(tokens) == 0:
                continue
            w = np.exp(z - z.max())
            w /= w.sum()
            out[h] = w @ vh
    return out


# ---------------------------------------------------------------------------
# The whole decode step
# ---------------------------------------------------------------------------
def decode_step(batch, rows=None, scores_fp32: np.ndarray | None = None) -> dict:
    """metadata -> scores -> selection -> table/ctx -> attention, for ``rows``
    (default: all rows).

    The selection is a floating-point decision; it is taken on float32 scores
    (the precision of the device kernel's accumulator). ``scores_fp32`` lets a
    caller pass the device's own float32 block scores so that the selection,
    table and context lengths can be compared bit for bit."""
    meta = build_metadata(batch.seq_lens, batch.query_lens)
    N = len(meta["row_req"])
    rows = list(range(N)) if rows is None else [int(r) for r in rows]
    if scores_fp32 is None:
        s64 = block_scores(batch.index_q, batch.index_k, batch.block_table, batch.seq_lens,
                           batch.query_lens, batch.ld_s, rows=rows,
                           index_scale=getattr(batch, "index_scale", None))
        s32 = s64.astype(np.float32)
    else:
        s64 = None
        s32 = np.asarray(scores_fp32, dtype=np.float32)
    topk = batch.topk
    sel_out = np.full((N, topk), -1, dtype=np.int64)
    table = np.zeros((N, SUBS_PER_PAGE * topk), dtype=np.int64)
    ctx = np.zeros(N, dtype=np.int64)
    out = np.zeros((N, batch.num_q_heads, batch.q.shape[-1]), dtype=np.float64)
    for n in rows:
        r = int(meta["row_req"][n])
        v = visible_keys(meta["row_pos"][n])
        nb = num_blocks(v)
        sel = select_blocks(s32[n].astype(np.float64), nb, topk)
        sel_out[n] = selection_row_outputs(sel, topk)
        table[n] = sparse_table_row(sel, batch.block_table[r], topk)
        ctx[n] = context_length(sel, v)
        out[n] = sparse_attention_row(batch.q[n], batch.k_cache, batch.v_cache, batch.kv_dtype,
                                      batch.scale_mode, batch.k_scale, batch.v_scale,
                                      batch.block_table[r], sel, v, batch.sm_scale)
    return {"meta": meta, "scores": s64, "scores_fp32": s32, "sel": sel_out,
            "table": table, "ctx": ctx, "out": out, "rows": rows}


def _table_keys_values(batch, table: np.ndarray, n: int, c: int, g: int):
    """Dequantised K and V [c][128] of row n's tokens u < c for KV head g,
    walked through the page-16 table (entry u // 16 names the sub-page of
    token u, slot u % 16)."""
    kh = np.empty((c, 128))
    vh = np.empty((c, 128))
    dec = bf16_to_f64 if batch.kv_dtype == 0 else e4m3fn_to_f64
    for u in range(c):
        sub = int(table[n][u // SUB])
        slot = u % SUB
        ks = vs = 1.0
        if batch.scale_mode == 1:
            ks = float(batch.k_scale.reshape(-1)[0])
            vs = float(batch.v_scale.reshape(-1)[0])
        elif batch.scale_mode == 2:
            ks = float(batch.k_scale[sub, slot, g])
            vs = float(batch.v_scale[sub, slot, g])
        kh[u] = ks * dec(tile_row(batch.k_cache[sub, g], slot))
        vh[u] = vs * dec(batch.v_cache[sub, g, :, slot])
    return kh, vh


def attention_from_table(batch, table: np.ndarray, ctx: np.ndarray, rows) -> np.ndarray:
    """Attention for given rows driven by a page-16 table and context lengths
    (the path's own contract: entry u // 16 of the row names the sub-page of
    token u, slot u % 16). Used to check the device's attention on the device's
    own table, so selection near-ties do not mix into attention error."""
    out = np.zeros((len(rows), batch.num_q_heads, batch.q.shape[-1]), dtype=np.float64)
    hkv_n = batch.k_cache.shape[1]
    group = batch.num_q_heads // hkv_n
    for i, n in enumerate(rows):
        c = int(ctx[n])
        q = bf16_to_f64(batch.q[n])
        for g in range(hkv_n):
            kh, vh = _table_keys_values(batch, table, n, c, g)
            out[i, g * group:(g + 1) * group] = softmax_attention(
                q[g * group:(g + 1) * group], kh, vh, batch.sm_scale)
    return out


def attention_lse_from_table(batch, table: np.ndarray, ctx: np.ndarray, rows,
                             sinks: np.ndarray | None = None):
    """As attention_from_table, also returning the natural-log LSE per (row,
    head) and applying optional per-query-head sinks [Hq] ([P3] 实现拆解
    items 1-2; see softmax_attention_lse). Returns (out [R][Hq][128],
    lse [R][Hq])."""
    out = np.zeros((len(rows), batch.num_q_heads, batch.q.shape[-1]), dtype=np.float64)
    lse = np.full((len(rows), batch.num_q_heads), -np.inf)
    hkv_n = batch.k_cache.shape[1]
    group = batch.num_q_heads // hkv_n
    for i, n in enumerate(rows):
        c = int(ctx[n])
        q = bf16_to_f64(batch.q[n])
        for g in range(hkv_n):
            kh, vh = _table_keys_values(batch, table, n, c, g)
            hs = slice(g * group, (g + 1) * group)
            out[i, hs], lse[i, hs] = softmax_attention_lse(
                q[hs], kh, vh, batch.sm_scale, None if sinks is None else np.asarray(sinks)[hs])
    return out, lse


# ---------------------------------------------------------------------------
# The step before the path: new tokens written into the paged caches
# ([P1] 实现拆解 items 1, 2 and 5: the fused K/V insert writes the separate K
# and V planes and, unless the layer reuses another layer's index, the index
# cache; FP8 caches carry per-token-head or scalar K/V scales)
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0   # largest finite e4m3fn magnitude


def tile_store(tile: np.ndarray, tok: int, row: np.ndarray) -> None:
    """Inverse of tile_row: element d of the token goes to [d//32][(d//8)%4][tok][d%8]."""
    tile[:, :, tok, :] = np.asarray(row).reshape(4, 4, 8)


def _f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16).copy()


def _f32_to_e4m3fn_codes(x32: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy().copy()


def quantize_row(x_bits: np.ndarray, kv_dtype: int, scale_mode: int, scalar_scale: float | None):
    """Stored values and scale of one token-head row of 128 bf16 inputs, in
    fp32 (each code is decided in fp32, as the device decides it):
      per-token-head scale: s = fp32(max |x|) / 448, or 1 for an all-zero row
        (bf16 storage keeps s = 1);
      scalar scale: s = the given fp32 scale; no scale: s = 1;
      fp8: code = e4m3fn RNE of clamp(fp32(x) / s, -448, 448);
      bf16: stored = bf16 RNE of fp32(x) / s.
    So that s x stored reproduces x up to the storage format's rounding."""
    x = bf16_to_f64(np.asarray(x_bits)).astype(np.float32)
    if scale_mode == 2 and kv_dtype == 1:
        amax = np.float32(np.max(np.abs(x)))
        s = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    elif scale_mode == 1:
        s = np.float32(scalar_scale)
    else:
        s = np.float32(1.0)
    y = (x / s).astype(np.float32)
    if kv_dtype == 1:
        y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
        return _f32_to_e4m3fn_codes(y), float(s)
    return _f32_to_bf16_bits(y), float(s)


def cache_insert(k_cache, v_cache, k_scale, v_scale, index_k, slot_mapping, k_new, v_new,
                 index_k_new, kv_dtype: int, scale_mode: int):
    """Writes token t of k_new / v_new ([T][Hkv][128] bf16) and index_k_new
    ([T][128] bf16, or None to leave the index cache alone) at slot
    slot_mapping[t] = 128 * page + offset (negative, or past the caches' last
    page: skipped). Returns updated
    copies (k_cache, v_cache, k_scale, v_scale, index_k). Per-token-head scales
    are written for every inserted token-head; a scalar scale is only read."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    ks = None if k_scale is None else np.array(k_scale, dtype=np.float32, copy=True)
    vs = None if v_scale is None else np.array(v_scale, dtype=np.float32, copy=True)
    ik = None if index_k is None else np.array(index_k, copy=True)
    hkv_n = kc.shape[1]
    num_slots = PAGE * (kc.shape[0] // SUBS_PER_PAGE)
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0 or slot >= num_slots:
            continue
        page, off = divmod(int(slot), PAGE)
        sub, j = SUBS_PER_PAGE * page + off // SUB, off % SUB
        for h in range(hkv_n):
            for plane, cache, scales, new in (("k", kc, ks, k_new), ("v", vc, vs, v_new)):
                scalar = None if scales is None or scale_mode != 1 else float(scales.reshape(-1)[0])
                stored, s = quantize_row(np.asarray(new)[t, h], kv_dtype, scale_mode, scalar)
                if plane == "k":
                    tile_store(cache[sub, h], j, stored)
                else:
                    cache[sub, h, :, j] = stored
                if scale_mode == 2:
                    scales.reshape(-1, SUB, hkv_n)[sub, j, h] = np.float32(s)
        if index_k_new is not None and ik is not None:
            tile_store(ik[page, off // SUB], j, np.asarray(index_k_new)[t])
    return kc, vc, ks, vs, ik


def index_insert_fp8(index_k_codes, index_scale, slot_mapping, index_k_new):
    """The index half of the insert for an FP8 index cache: token t's index
    key ([T][128] bf16) is quantised with its own scale by the per-token rule
    of quantize_row (s = fp32(max |x|) / 448, 1 for an all-zero row; code =
    e4m3fn RNE of clamp(x / s, +-448)), stored at slot_mapping[t] = 128 * page
    + offset (negative, or past the last page: skipped) with index_scale[page]
    [offset] = s. Returns updated copies (index_k_codes, index_scale)."""
    ik = np.array(index_k_codes, copy=True)
    isc = np.array(index_scale, dtype=np.float32, copy=True)
    num_slots = PAGE * ik.shape[0]
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0 or slot >= num_slots:
            continue
        page, off = slot // PAGE, slot % PAGE
        codes, sc = quantize_row(np.asarray(index_k_new)[t], 1, 2, None)
        tile_store(ik[page, off // SUB], off % SUB, codes)
        isc[page, off] = np.float32(sc)
    return ik, isc

/*
 * msa.h — C ABI of the block-sparse paged decode-attention library for AMD
 * MI355X (gfx950).
 *
 * The method (MiniMax-M3-style sparse attention) is described on the
 * prhub.com.cn summaries of vLLM pull requests, cited below by PR number and the
 * page's own section names:
 *   #47287  ROCm AITER sparse paged attention for MiniMax-M3
 *   #54682  gfx950 decode index scoring and top-k
 *   #56170  cu_seqlens_k first element zeroed on the device
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked (host). The caller owns every
 *     buffer, including the workspace; the library allocates nothing and keeps
 *     no state except a per-device cached compute-unit count and, for
 *     msa_sparse_decode_static, its fixed per-device workspace array and that
 *     array's address on each device.
 *   - Calls only enqueue kernels on `stream` (a hipStream_t; NULL = the null
 *     stream) and return. They never copy between host and device and never
 *     synchronise, so they can be captured into a HIP graph.
 *   - Host-checkable problems (null required pointer, unsupported shape, small
 *     workspace) return an error status and enqueue nothing.
 *   - Device data is not validated, but every kernel clamps what it reads from
 *     device arrays (lengths, table entries, page ids) so that malformed data
 *     gives wrong numbers rather than out-of-bounds accesses.
 *   - Fixed sizes: 128-token KV / index-K pages = 128-token sparse blocks, a
 *     page-16 view (8 sub-pages per page), head dim 128, index dim 128, one KV
 *     head and one index head.
 *
 * Data layouts (all row-major, innermost last)
 *   A "tile" is 16 tokens x 128 dims stored MFMA-shuffled as [4][4][16][8]:
 *   (32-dim chunk, 8-dim group, token, element); dim d of token t is at
 *   [d/32][(d%32)/8][t][d%8], so each 64-lane MFMA operand is one contiguous
 *   run in memory.
 *   index_q      [N][128]                bf16
 *   index_k      [P][8][4][4][16][8]     bf16   page, 16-token tile, shuffled tile
 *   q, out       [N][Hq][128]            bf16
 *   k_cache      [8P][Hkv][4][4][16][8]  bf16 | fp8 e4m3fn   one shuffled tile per sub-page
 *   v_cache      [8P][Hkv][128][16]      bf16 | fp8 e4m3fn   dim-major sub-pages
 *   k/v_scale    scalar: [1] fp32;  per-token-head: [8P][16][Hkv] fp32
 *   block_table  [R][ld_bt]              int32  physical page-128 ids
 *   block_scores [N][ld_s]               fp32
 *   sparse_table [N][ld_table]           int32  page-16 sub-page ids
 *   Sub-page i of physical page p is 8*p + i. Token t of a request lives in
 *   page block_table[r][t / 128], slot s = t % 128: tile s / 16 of the index-K
 *   page, sub-page 8*page + s / 16 of the K/V caches, token s % 16 there.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* msa_stream_t; /* a hipStream_t */

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = -1, /* null required pointer, negative size, bad enum */
  MSA_ERR_UNSUPPORTED = -2, /* shape outside what the kernels implement */
  MSA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  MSA_ERR_HIP = -4          /* a launch failed (hipGetLastError) */
} msa_status;

typedef enum { MSA_KV_BF16 = 0, MSA_KV_FP8_E4M3FN = 1 } msa_kv_dtype;

typedef enum {
  MSA_SCALE_NONE = 0,          /* K-hat = K, V-hat = V (bf16 caches) */
  MSA_SCALE_SCALAR = 1,        /* one fp32 scale for K and one for V */
  MSA_SCALE_PER_TOKEN_HEAD = 2 /* one fp32 scale per (token, KV head) */
} msa_scale_mode;

enum {
  MSA_PAGE_TOKENS = 128,
  MSA_SUBPAGE_TOKENS = 16,
  MSA_HEAD_DIM = 128,
  MSA_INDEX_DIM = 128,
  MSA_MAX_REQS = 4096,      /* requests per batch */
  MSA_MAX_Q_HEADS = 128,    /* query heads sharing the one KV head */
  MSA_MAX_TOPK = 8192,      /* selected blocks per row */
  MSA_MAX_SEQ_LEN = 1048576, /* tokens per request (8192 blocks) */
  MSA_MAX_PAGES = 16777216,  /* physical pages P (int32 slots 128*page + offset; 8*P sub-page ids) */
  MSA_SCORE_ROWS_PER_UNIT = 64, /* query rows of one request scored per work unit */
  MSA_STATIC_SCRATCH_BYTES = 33554432 /* workspace of msa_sparse_decode_static: 32 MiB per device */
};

/*
 * Batch description: host struct holding device pointers and host scalars.
 * Decode requests come first and prefill requests after (#56170 page,
 * 关键源码片段), though nothing here depends on that order.
 */
typedef struct msa_batch {
  const int32_t* seq_lens;    /* [num_reqs] L_r: KV tokens incl. this step's new ones */
  const int32_t* query_lens;  /* [num_reqs] ql_r: query rows, 0 <= ql_r <= L_r */
  const int32_t* block_table; /* [num_reqs][ld_bt] page-128 physical ids */
  /* outputs of msa_build_metadata, inputs of the other calls */
  int32_t* cu_seqlens_q;      /* [num_reqs+1] 0, ql_0, ql_0+ql_1, ... */
  int32_t* cu_seqlens_k;      /* [num_reqs+1] 0, L_0, L_0+L_1, ... */
  int32_t* cu_blocks;         /* [num_reqs+1] prefix of ceil(L_r/128) */
  int32_t* cu_units;          /* [num_reqs+1] prefix of ceil(L_r/128)*ceil(ql_r/64):
                                 the score kernel's work units */
  int32_t* row_req;           /* [num_rows] request id of each query row */
  int32_t* row_pos;           /* [num_rows] absolute position L_r - ql_r + i */
  int32_t num_reqs;           /* host, exact */
  int32_t num_rows;           /* host, exact: sum of query_lens */
  int32_t ld_bt;              /* host: row stride of block_table (>= blocks of any request) */
  int32_t max_seq_len;        /* host: upper bound of every seq_len (sizes grids) */
  int32_t num_pages;          /* host: P <= MSA_MAX_PAGES, physical pages in index_k / k_cache / v_cache */
} msa_batch;

/* K/V cache description (host struct with device pointers). Slots of a
 * request's pages at or past its seq_len (the rest of its last page) are
 * never visible and may hold any bits, NaN codes and NaN scales included, in
 * the K/V caches, their scales and the index cache: no output depends on them. */
typedef struct msa_kv {
  const void* k_cache;   /* [8P][Hkv][4][4][16][8] */
  const void* v_cache;   /* [8P][Hkv][128][16] */
  const float* k_scale;  /* NULL (MSA_SCALE_NONE), [1] or [8P][16][Hkv] */
  const float* v_scale;
  int32_t kv_dtype;      /* msa_kv_dtype */
  int32_t scale_mode;    /* msa_scale_mode; MSA_SCALE_NONE requires bf16 */
  int32_t num_kv_heads;  /* must be 1 */
  int32_t num_pages;     /* P <= MSA_MAX_PAGES: the caches hold 8P sub-pages */
} msa_kv;

/*
 * msa_build_metadata — device-side batch metadata with no host round trip
 * (#56170 page, 实现拆解 items 1-3 and 关键源码片段: cu_seqlens_k is a zero
 * followed by the running sum of seq_lens, written on the device; prefill rows
 * get a request id and an absolute position).
 * Writes cu_seqlens_q, cu_seqlens_k, cu_blocks, cu_units, row_req, row_pos.
 * Errors: INVALID_ARG for null pointers or num_reqs/num_rows < 0;
 * UNSUPPORTED for num_reqs > MSA_MAX_REQS, max_seq_len > MSA_MAX_SEQ_LEN or
 * num_pages > MSA_MAX_PAGES (every call taking a batch checks the same; every
 * call taking an msa_kv rejects num_pages > MSA_MAX_PAGES likewise).
 */
msa_status msa_build_metadata(msa_stream_t stream, const msa_batch* batch);

/*
 * msa_index_score — index scores pooled per 128-token block (#54682 page,
 * 功能与动机 and 实现拆解 item 1: the per-row decode scorer, with work mapped
 * to each request's real block count and index-K tiles shared by a request's
 * rows).
 *   block_scores[n][b] = max over visible tokens t of block b (t <= row_pos[n])
 *                        of dot(index_q[n], index_k[token t]),  b < nb_n
 *   block_scores[n][b] = -inf for nb_n <= b < ld_s,  nb_n = ceil((row_pos[n]+1)/128)
 * Reads seq_lens / query_lens directly (the metadata arrays are not needed).
 * index_q [N][128] bf16, index_k [P][8][4][4][16][8] bf16 (see the layouts
 * above), block_scores [N][ld_s] fp32.
 * Errors: INVALID_ARG for null pointers; UNSUPPORTED if ld_s < ceil(max_seq_len/128).
 */
msa_status msa_index_score(msa_stream_t stream, const msa_batch* batch, const void* index_q,
                           const void* index_k, float* block_scores, int32_t ld_s);

/*
 * msa_topk_block_table — fused top-k selection, page-16 sparse block table and
 * context lengths (#54682 page, 实现拆解 items 1 and 4; #47287 page, 实现拆解
 * item 3 and 评论区精华 on keeping the zero padding inside the row).
 * Requires row_req / row_pos from msa_build_metadata (or msa_sparse_decode).
 * For each row n with nb_n eligible blocks, K' = min(topk, nb_n) blocks are kept
 * under the total order (score descending, block id ascending, -0 == +0) and
 * listed by ascending block id b_0 < ... < b_{K'-1}:
 *   sparse_table[n][8j+i] = 8*block_table[r][b_j] + i   (j < K', i < 8)
 *   sparse_table[n][m]    = 0                            (8K' <= m < 8*topk)
 *   ctx_lens[n]           = sum_j min(128, row_pos[n]+1 - 128*b_j)
 *   sel_blocks[n][j]      = b_j, then -1                 (optional, may be NULL)
 * Nothing is written at or past column 8*topk of sparse_table (its row stride
 * is 8*topk).
 * Errors: INVALID_ARG for null required pointers or topk < 1; UNSUPPORTED for
 * topk > MSA_MAX_TOPK or ld_s < ceil(max_seq_len/128).
 */
msa_status msa_topk_block_table(msa_stream_t stream, const msa_batch* batch,
                                const float* block_scores, int32_t ld_s, int32_t topk,
                                int32_t* sparse_table, int32_t* ctx_lens, int32_t* sel_blocks);

/*
 * msa_sparse_paged_attn — paged attention over a page-16 sparse table with an
 * online softmax (#47287 page, 功能与动机: attention over a few selected logical
 * blocks; 实现拆解 item 2: FP8 k_scale / v_scale, scalar or per-token-head;
 * 实现拆解 item 3: the page-16 view of the page-128 cache).
 * Row n, query head h (KV head 0): tokens u < ctx_lens[n] live in sub-page
 * sparse_table[n][u/16], slot u%16;
 *   out[n][h] = sum_u softmax_u(sm_scale * q[n][h] . K-hat_u) V-hat_u
 * with K-hat = k_scale * K, V-hat = v_scale * V. Rows with ctx 0 give zeros.
 * Output is bf16 (round to nearest even). Also serves a selection reused from
 * another layer: the table need not come from msa_topk_block_table.
 *   max_ctx (host): upper bound of ctx_lens; larger device values are clamped.
 *   ld_table: row stride of sparse_table, >= ceil(max_ctx/16).
 *   workspace: >= msa_workspace_bytes(num_rows, num_q_heads, max_ctx, 0) bytes,
 *   256-byte aligned; its contents need no initialisation; may be NULL when
 *   that size is 0 (every row fits one split).
 * Errors: INVALID_ARG for null required pointers or sizes < 0; UNSUPPORTED for
 * num_kv_heads != 1, num_q_heads > MSA_MAX_Q_HEADS, max_ctx > MSA_MAX_SEQ_LEN,
 * bad dtype/scale pairing (MSA_SCALE_NONE with fp8), or a launch whose grid
 * (rows x head groups x token splits, or rows x query heads) would pass 2^31
 * workgroups; WORKSPACE if the workspace is too small.
 */
msa_status msa_sparse_paged_attn(msa_stream_t stream, const void* q, int32_t num_rows,
                                 int32_t num_q_heads, const msa_kv* kv,
                                 const int32_t* sparse_table, int32_t ld_table,
                                 const int32_t* ctx_lens, int32_t max_ctx, float sm_scale,
                                 void* out, void* workspace, size_t workspace_bytes);

/*
 * msa_sparse_decode — the whole decode step on one stream with no host
 * synchronisation: metadata, index score + pooling, top-k + page-16 table +
 * context lengths, sparse paged attention and the split merge (#54682 page,
 * 实现拆解 items 2-3: the indexer's selection and sparse table feed attention
 * in the same step). Three launches: index scores, the selection fused into
 * attention, the split merge (a second scoring launch for batches of more
 * than 64 rows; no merge when every row fits one split). No state is carried
 * between calls, so the step can be captured in a HIP graph and replayed. Also writes the batch
 * metadata arrays (as msa_build_metadata does).
 *   sparse_table [N][8*topk], ctx_lens [N]: written (outputs of the top-k step).
 *   sel_blocks [N][topk]: optional (NULL skips it).
 *   block_scores [N][ld_s]: optional; when NULL the scores live in the
 *   workspace. ld_s >= ceil(max_seq_len/128).
 *   workspace: >= msa_workspace_bytes(num_rows, num_q_heads, 128*topk,
 *   block_scores ? 0 : ld_s) bytes (NULL allowed when that is 0).
 *   Launches of 2048 to 262144 rows (prefill-sized) given a workspace of
 *   msa_decode_workspace_bytes(num_rows, max_seq_len, num_q_heads, topk,
 *   block_scores ? 0 : ld_s) bytes take the block-major path instead: the
 *   top-k step runs on its own and also leaves each row's selection as bit
 *   words; when the batch has at most 16384 (request, block) pairs the rows
 *   that chose each block are counted (one more launch) and the attention
 *   grid is balanced by (row, block) pairs rather than blocks; the
 *   workgroups attend the rows that chose a block from one copy of the
 *   block's K/V, and the per-block partials are merged (5 or 6 launches:
 *   two scoring launches, top-k, the optional count, attention, merge). Each partial
 *   keeps its max and sum in fp32 and its 16x128 accumulator in fp16, scaled by a power of two so that its
 *   largest magnitude is below 1: from the accumulator itself, or, for bf16
 *   K/V with no scales, from the bound 128 * max|V| of the block (the error
 *   this adds to an output is at most about 2^-11 of the largest |V| entry
 *   of the blocks the row attends). Same results up to that and rounding
 *   order; with the smaller workspace the per-row path runs.
 * Errors: union of the errors of the steps.
 */
msa_status msa_sparse_decode(msa_stream_t stream, const msa_batch* batch, const void* index_q,
                             const void* index_k, const void* q, int32_t num_q_heads,
                             const msa_kv* kv, int32_t topk, float sm_scale, void* out,
                             int32_t* sparse_table, int32_t* ctx_lens, int32_t* sel_blocks,
                             float* block_scores, int32_t ld_s, void* workspace,
                             size_t workspace_bytes);

/*
 * The _ex entry points — the same operations with optional extras; each plain
 * entry point is its _ex form with every extra NULL.
 *
 * FP8 index cache (index_k_scale != NULL; the optional FP8 index storage and
 * FP8 decode scoring named on the #54682 page, 相关 PRs): index_k then holds
 * e4m3fn codes [P][8][4][4][16][8] u8 (the bf16 layout, one byte per value:
 * 16 KiB a page) and index_k_scale [P][128] fp32 one scale per token slot;
 * token t's key is index_k_scale[page][t%128] * e4m3fn(code). The index query
 * stays bf16; each token's score is its scale times the dot product of the
 * query with the codes' values (exact bf16 products, fp32 sum).
 *
 * Sinks and LSE (#54404 page, 实现拆解 item 1: a decode operator that also
 * returns the natural-log LSE, for merging partial attention; item 2: one
 * learnable float32 sink per query head):
 *   sinks [num_q_heads] fp32 (device), or NULL: head h's softmax denominator
 *     gains exp(sinks[h]) — a logit with no value vector —
 *       out[n][h] = sum_u e^{z_u} V-hat_u / (e^{sinks[h]} + sum_u e^{z_u}),
 *     z_u = sm_scale * q[n][h] . K-hat_u. -inf means no sink; +inf gives zeros.
 *   lse [num_rows][num_q_heads] fp32 (device), or NULL: written with
 *     ln sum_u e^{z_u} over the attended tokens; the sink is not included, so
 *     partial results over disjoint token sets can be merged with it and a
 *     sink applied once afterwards. Rows with ctx 0 get -inf (and zero output).
 * No extra workspace; errors as for the plain entry points.
 */
msa_status msa_index_score_ex(msa_stream_t stream, const msa_batch* batch, const void* index_q,
                              const void* index_k, const float* index_k_scale,
                              float* block_scores, int32_t ld_s);
msa_status msa_sparse_paged_attn_ex(msa_stream_t stream, const void* q, int32_t num_rows,
                                    int32_t num_q_heads, const msa_kv* kv,
                                    const int32_t* sparse_table, int32_t ld_table,
                                    const int32_t* ctx_lens, int32_t max_ctx, float sm_scale,
                                    const float* sinks, void* out, float* lse, void* workspace,
                                    size_t workspace_bytes);
msa_status msa_sparse_decode_ex(msa_stream_t stream, const msa_batch* batch, const void* index_q,
                                const void* index_k, const float* index_k_scale, const void* q,
                                int32_t num_q_heads, const msa_kv* kv, int32_t topk,
                                float sm_scale, const float* sinks, void* out, float* lse,
                                int32_t* sparse_table, int32_t* ctx_lens, int32_t* sel_blocks,
                                float* block_scores, int32_t ld_s, void* workspace,
                                size_t workspace_bytes);

/*
 * msa_sparse_decode_static — msa_sparse_decode_ex with no workspace argument
 * and no allocation, for callers that cannot call hipMalloc (code under HIP
 * graph capture, tight serving loops, harnesses that forbid it). The
 * workspace is a fixed device array of MSA_STATIC_SCRATCH_BYTES inside the
 * library, one per device, held from the library's load until the process
 * ends; its address on the current device is looked up (hipGetSymbolAddress)
 * on the first call made with that device current. Results are those of
 * msa_sparse_decode_ex given a workspace of MSA_STATIC_SCRATCH_BYTES bytes
 * (the same path is chosen). Nothing in it needs clearing: every byte a call
 * reads was written earlier in the same call.
 * Every call on one device shares that device's array: calls that may
 * overlap on one device (two streams, or two host threads) race and must be
 * serialised by the caller.
 * Errors: as msa_sparse_decode_ex; WORKSPACE when the call needs more than
 * MSA_STATIC_SCRATCH_BYTES, i.e. msa_workspace_bytes(num_rows, num_q_heads,
 * 128*topk, block_scores ? 0 : ld_s) > MSA_STATIC_SCRATCH_BYTES (pass
 * block_scores to keep the scores out of it); HIP if the array's address
 * cannot be obtained.
 */
msa_status msa_sparse_decode_static(msa_stream_t stream, const msa_batch* batch, const void* index_q,
                                    const void* index_k, const float* index_k_scale, const void* q,
                                    int32_t num_q_heads, const msa_kv* kv, int32_t topk,
                                    float sm_scale, const float* sinks, void* out, float* lse,
                                    int32_t* sparse_table, int32_t* ctx_lens, int32_t* sel_blocks,
                                    float* block_scores, int32_t ld_s);

/*
 * msa_cache_insert — the step before the path: writes new tokens' K, V and
 * index keys into the paged caches (#47287 page, 实现拆解 items 1, 2 and 5: the
 * fused K/V insert fills the separate K and V planes and, unless the layer
 * reuses another layer's index, the index cache; FP8 caches carry
 * per-token-head or scalar K/V scales).
 *   slot_mapping [num_tokens] int32: 128*page + offset of token t in its
 *     page-128 physical page; negative (or >= 128*kv->num_pages): skipped.
 *   k_new, v_new [num_tokens][Hkv][128] bf16.
 *   kv: the caches written, in the layouts above; with
 *     MSA_SCALE_PER_TOKEN_HEAD the scale arrays [8P][16][Hkv] are written too
 *     (the struct's pointers are written through).
 *   index_k_new [num_tokens][128] bf16, or NULL to leave the index cache alone
 *     (a layer that reuses another layer's index); index_k [P][8][4][4][16][8]
 *     bf16 is then written.
 * Quantisation, each code decided in fp32: e4m3fn with per-token-head scales
 * stores code = RNE(clamp(x / s, -448, 448)) with s = max|x| / 448 over the
 * token-head (1 for an all-zero row); with a scalar scale s is read from
 * k_scale[0] / v_scale[0] and not written; bf16 caches store RNE(x / s) with
 * s = 1 unless scalar (per-token-head bf16 caches get scale 1).
 * Two tokens mapped to one slot race. One launch, no workspace.
 * Errors: as check of kv in msa_sparse_paged_attn; INVALID_ARG for
 * num_tokens < 0, null slot_mapping / k_new / v_new, or index_k_new without
 * index_k.
 */
msa_status msa_cache_insert(msa_stream_t stream, int32_t num_tokens, const int32_t* slot_mapping,
                            const void* k_new, const void* v_new, const msa_kv* kv,
                            const void* index_k_new, void* index_k);
/*
 * msa_cache_insert_ex — msa_cache_insert with index_k_scale [P][128] fp32:
 * when it is non-NULL (and index_k_new is given) the index cache is the FP8
 * one described above, and each token's index key is stored by the
 * per-token rule s = max|x| / 448 over its 128 values (1 for an all-zero
 * row), codes e4m3fn RNE of clamp(x / s, -448, 448), s written to
 * index_k_scale[page][offset]. NULL: the bf16 copy of msa_cache_insert.
 */
msa_status msa_cache_insert_ex(msa_stream_t stream, int32_t num_tokens,
                               const int32_t* slot_mapping, const void* k_new, const void* v_new,
                               const msa_kv* kv, const void* index_k_new, void* index_k,
                               float* index_k_scale);

/*
 * msa_workspace_bytes — workspace needed by msa_sparse_paged_attn (ld_s = 0)
 * or msa_sparse_decode (max_ctx = 128*topk; ld_s > 0 when the scores live in
 * the workspace) on the current device. Returns 0 for invalid arguments.
 */
size_t msa_workspace_bytes(int32_t num_rows, int32_t num_q_heads, int32_t max_ctx, int32_t ld_s);

/*
 * msa_decode_workspace_bytes — workspace that lets msa_sparse_decode(_ex)
 * take the block-major path on launches of 2048 to 262144 rows (the batch's
 * num_rows and max_seq_len): per row, num_q_heads/16 (rounded up) x topk
 * partials of 4224 bytes and one 8-byte selection word per 32 blocks of
 * ceil(max_seq_len/128); 64 KiB of per-block row counts; and the scores when
 * ld_s > 0. For other row counts
 * it equals msa_workspace_bytes(num_rows, num_q_heads, 128*topk, ld_s).
 * Returns 0 for invalid arguments.
 */
size_t msa_decode_workspace_bytes(int32_t num_rows, int32_t max_seq_len, int32_t num_q_heads, int32_t topk,
                                  int32_t ld_s);

/* Human-readable name of a status code (static storage). */
const char* msa_status_string(msa_status status);

/* Library ABI version: major*10000 + minor*100 + patch. */
int32_t msa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */

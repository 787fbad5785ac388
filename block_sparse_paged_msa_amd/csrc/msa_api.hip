// Host side of the C ABI declared in include/msa.h: argument validation,
// launch policy (grid sizes from host-known bounds and the device's compute
// unit count), workspace layout and the stream-ordered launches. No call here
// allocates, copies between host and device, or synchronises.
#include <atomic>
#include <climits>
#include <mutex>

#include "msa.h"
#include "msa_kernels.h"

// Workspace of msa_sparse_decode_static, for callers that cannot allocate:
// one fixed array per device, loaded with the library's code object and held
// until the process ends. Host code never uses its name as an address (on
// the host it is only a stand-in for the symbol); the device address comes
// from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[MSA_STATIC_SCRATCH_BYTES];

namespace {

using msa::kDim;
using msa::kHeadTile;
using msa::kPage;
using msa::kRowsPerUnit;
using msa::kSub;

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int c = g_cu_count[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  g_cu_count[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept.
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Attention split policy: the smallest split (64 tokens times a power of two,
// at most kMaxSplitTokens) whose workgroup count stays within two workgroups
// per compute unit, so that short batches still spread over the whole chip
// while long ones keep few partials.
struct AttnPlan {
  int hgroups;
  int split_tok;
  int nsplit;
};

AttnPlan attn_plan(int num_rows, int num_q_heads, int max_ctx) {
  AttnPlan p;
  p.hgroups = static_cast<int>(ceil_div(num_q_heads, kHeadTile));
  const int64_t ctx = max_ctx < 1 ? 1 : max_ctx;
  const int64_t target = 2LL * cu_count();
  // from 64 tokens (one sub-page per wave) up: short rows in small batches
  // get twice the workgroups that 128-token splits give (bf16 decode batch,
  // 8 rows of 2048 selected tokens: 128 -> 256 workgroups, 20.35 -> 20.04 us)
  int64_t split = 64;
  while (split < ctx && split < kMaxSplitTokens &&
         static_cast<int64_t>(num_rows) * p.hgroups * ceil_div(ctx, split) > target)
    split *= 2;
  p.split_tok = static_cast<int>(split);
  p.nsplit = static_cast<int>(ceil_div(ctx, split));
  return p;
}

// A per-row launch whose attention grid (rows x head groups x token splits)
// or, when rows are split, merge grid (rows rounded up to 8 x query heads)
// would not fit 31 bits is refused before anything is enqueued.
bool attn_grid_fits(int num_rows, int num_q_heads, int max_ctx) {
  const AttnPlan p = attn_plan(num_rows, num_q_heads, max_ctx);
  const int64_t attn = static_cast<int64_t>(num_rows) * p.hgroups * p.nsplit;
  const int64_t merge = p.nsplit > 1 ? (static_cast<int64_t>(num_rows) + 7) / 8 * 8 * num_q_heads : 0;
  return attn <= INT32_MAX && merge <= INT32_MAX;
}

struct WsLayout {
  size_t partials, scores, total;
};

// Workspace: split partials (rows with several splits) then, for the fused
// step without a caller score buffer, the block scores.
WsLayout ws_layout(int num_rows, int num_q_heads, int max_ctx, int ld_s) {
  const AttnPlan p = attn_plan(num_rows, num_q_heads, max_ctx);
  WsLayout w;
  size_t off = 0;
  w.partials = off;
  // one slot per (row, head group, split): m[16], l[16] fp32 + fp16 acc[16][128]
  if (p.nsplit > 1)
    off += align256(static_cast<size_t>(num_rows) * p.hgroups * p.nsplit *
                    (sizeof(float) * 2 * kHeadTile + sizeof(uint16_t) * kHeadTile * kDim));
  w.scores = off;
  if (ld_s > 0) off += align256(sizeof(float) * static_cast<size_t>(num_rows) * ld_s);
  w.total = off;
  return w;
}

// Block-major attention for the fused step (launches of at least this many
// rows, given the larger workspace): block partials for every row's topk
// slots, the selected block ids, then the scores as above.
constexpr int32_t kBlockMajorRows = 2048;
constexpr int32_t kBlockMajorMaxRows = 1 << 18;  // rows fit the row field of a list entry
// Launches of at most this many (request, block) items count each item's
// rows and balance the block-major grid by entries (one 4-byte count per
// item in the workspace); larger ones hand out items by grid stride.
constexpr int64_t kBalancedItemsMax = 16384;

struct BmLayout {
  size_t partials, words, counts, scores, total;
};

// Block-major workspace: partial slots, each row's selection words (one
// 8-byte word per 32 blocks of ceil(max_seq_len / 128)), the per-item row
// counts, then the scores when the caller passes no score buffer.
int bm_words(int nbmax) { return (nbmax + 31) / 32; }

BmLayout bm_layout(int num_rows, int nbmax, int num_q_heads, int topk, int ld_s) {
  const size_t hgroups = static_cast<size_t>(ceil_div(num_q_heads, kHeadTile));
  BmLayout w;
  size_t off = 0;
  w.partials = off;
  // one slot per (row, head group, selected block): m[16], l[16] fp32 + fp16 acc[16][128]
  off += align256(static_cast<size_t>(num_rows) * hgroups * static_cast<size_t>(topk) *
                  (sizeof(float) * 2 * kHeadTile + sizeof(uint16_t) * kHeadTile * kDim));
  w.words = off;
  off += align256(sizeof(uint64_t) * static_cast<size_t>(num_rows) * bm_words(nbmax));
  w.counts = off;
  off += align256(sizeof(int32_t) * static_cast<size_t>(kBalancedItemsMax));
  w.scores = off;
  if (ld_s > 0) off += align256(sizeof(float) * static_cast<size_t>(num_rows) * ld_s);
  w.total = off;
  return w;
}

msa_status hip_status(hipError_t e) { return e == hipSuccess ? MSA_OK : MSA_ERR_HIP; }

msa_status check_batch(const msa_batch* b, bool need_meta_outputs) {
  if (!b) return MSA_ERR_INVALID_ARG;
  if (b->num_reqs < 0 || b->num_rows < 0 || b->max_seq_len < 0) return MSA_ERR_INVALID_ARG;
  if (b->num_reqs > MSA_MAX_REQS || b->max_seq_len > MSA_MAX_SEQ_LEN) return MSA_ERR_UNSUPPORTED;
  if (b->num_rows > 0 && b->num_reqs == 0) return MSA_ERR_INVALID_ARG;
  if (b->num_reqs == 0) return MSA_OK;
  if (b->ld_bt < 1 || b->num_pages < 1) return MSA_ERR_INVALID_ARG;
  if (!b->seq_lens || !b->query_lens || !b->block_table) return MSA_ERR_INVALID_ARG;
  if (need_meta_outputs && (!b->cu_seqlens_q || !b->cu_seqlens_k || !b->cu_blocks || !b->cu_units))
    return MSA_ERR_INVALID_ARG;
  if (need_meta_outputs && b->num_rows > 0 && (!b->row_req || !b->row_pos)) return MSA_ERR_INVALID_ARG;
  if (b->num_pages > MSA_MAX_PAGES) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

int blocks_bound(const msa_batch* b) { return static_cast<int>(ceil_div(b->max_seq_len, kPage)); }

msa_status check_kv(const msa_kv* kv) {
  if (!kv || !kv->k_cache || !kv->v_cache) return MSA_ERR_INVALID_ARG;
  if (kv->kv_dtype != MSA_KV_BF16 && kv->kv_dtype != MSA_KV_FP8_E4M3FN) return MSA_ERR_INVALID_ARG;
  if (kv->scale_mode < MSA_SCALE_NONE || kv->scale_mode > MSA_SCALE_PER_TOKEN_HEAD) return MSA_ERR_INVALID_ARG;
  if (kv->num_pages < 1) return MSA_ERR_INVALID_ARG;
  if (kv->num_pages > MSA_MAX_PAGES) return MSA_ERR_UNSUPPORTED;
  if (kv->num_kv_heads != 1) return MSA_ERR_UNSUPPORTED;
  if (kv->kv_dtype == MSA_KV_FP8_E4M3FN && kv->scale_mode == MSA_SCALE_NONE) return MSA_ERR_UNSUPPORTED;
  if (kv->scale_mode != MSA_SCALE_NONE && (!kv->k_scale || !kv->v_scale)) return MSA_ERR_INVALID_ARG;
  return MSA_OK;
}

int32_t len_cap(const msa_batch* b) {
  const int64_t cap = static_cast<int64_t>(kPage) * b->ld_bt;
  return static_cast<int32_t>(cap < b->max_seq_len ? cap : b->max_seq_len);
}

MsaMetaArgs meta_args(const msa_batch* b) {
  MsaMetaArgs m;
  m.seq_lens = b->seq_lens;
  m.query_lens = b->query_lens;
  m.cu_q = b->cu_seqlens_q;
  m.cu_k = b->cu_seqlens_k;
  m.cu_blocks = b->cu_blocks;
  m.cu_units = b->cu_units;
  m.row_req = b->row_req;
  m.row_pos = b->row_pos;
  m.num_reqs = b->num_reqs;
  m.num_rows = b->num_rows;
  m.len_cap = len_cap(b);
  return m;
}

msa_status launch_score(hipStream_t s, const msa_batch* b, const void* index_q, const void* index_k,
                        const float* index_scale, float* scores, int32_t ld_s, bool write_meta) {
  MsaScoreArgs a;
  a.index_q = static_cast<const uint16_t*>(index_q);
  a.index_k = index_k;
  a.index_scale = index_scale;
  a.block_table = b->block_table;
  a.seq_lens = b->seq_lens;
  a.query_lens = b->query_lens;
  a.scores = scores;
  a.cu_q = b->cu_seqlens_q;
  a.cu_k = b->cu_seqlens_k;
  a.cu_blocks = b->cu_blocks;
  a.cu_units = b->cu_units;
  a.row_req = b->row_req;
  a.row_pos = b->row_pos;
  a.ld_s = ld_s;
  a.ld_bt = b->ld_bt;
  a.num_reqs = b->num_reqs;
  a.num_rows = b->num_rows;
  a.num_pages = b->num_pages;
  a.len_cap = len_cap(b);
  a.write_meta = write_meta ? 1 : 0;
  // a launch that may hold a request of more than 64 rows leaves such
  // requests to the tile kernel, launched right after on the same stream
  const bool tiles = b->num_rows > kRowsPerUnit;
  a.skip_big = tiles ? 1 : 0;
  // first-group slots r*S + j, S = ceil(len_cap/128)
  const int64_t S = ceil_div(a.len_cap, kPage) > 0 ? ceil_div(a.len_cap, kPage) : 1;
  a.blocks_per_req = static_cast<int32_t>(S);
  const int64_t units = S * b->num_reqs;
  int64_t wgs = ceil_div(units, 4);
  // decode launches: up to one slot per wave for batches of up to 64 slots
  // per compute unit (a wave that takes a second slot waits a whole page
  // before requesting it: fp8 K/V batch, 11 x 1024 slots, score kernel
  // 36.5 -> 36.3 us); prefill-sized launches keep 8 workgroups per unit
  const int64_t cap = (tiles ? 8LL : 16LL) * cu_count();
  if (wgs > cap) wgs = cap;
  if (wgs < 1) wgs = 1;
  hipError_t e = msa_launch_score(a, static_cast<int>(wgs), s);
  if (e != hipSuccess || !tiles) return hip_status(e);
  int64_t twgs = msa_score_tile_items_bound(b->num_rows, S);
  const int64_t tcap = cu_count();  // one 512-thread workgroup per compute unit
  if (twgs > tcap) twgs = tcap;
  if (twgs < 1) twgs = 1;
  return hip_status(msa_launch_score_tile(a, static_cast<int>(twgs), s));
}

MsaTopkArgs topk_args(const msa_batch* b, const float* scores, int32_t ld_s, int32_t topk, int32_t* table,
                      int32_t* ctx, int32_t* sel) {
  MsaTopkArgs a = {};
  a.scores = scores;
  a.block_table = b->block_table;
  a.row_req = b->row_req;
  a.row_pos = b->row_pos;
  a.table = table;
  a.ctx = ctx;
  a.sel = sel;
  a.ld_s = ld_s;
  a.ld_bt = b->ld_bt;
  a.topk = topk;
  a.num_rows = b->num_rows;
  a.num_reqs = b->num_reqs;
  return a;
}

msa_status launch_topk(hipStream_t s, const msa_batch* b, const float* scores, int32_t ld_s, int32_t topk,
                       int32_t* table, int32_t* ctx, int32_t* sel) {
  return hip_status(msa_launch_topk(topk_args(b, scores, ld_s, topk, table, ctx, sel), s));
}

MsaAttnArgs attn_args(const void* q, int32_t num_rows, int32_t num_q_heads, const msa_kv* kv, int32_t ld_table,
                      int32_t max_ctx, float sm_scale, void* out, void* ws) {
  const AttnPlan p = attn_plan(num_rows, num_q_heads, max_ctx);
  const WsLayout w = ws_layout(num_rows, num_q_heads, max_ctx, 0);
  MsaAttnArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = kv->k_cache;
  a.v_cache = kv->v_cache;
  a.k_scale = kv->k_scale;
  a.v_scale = kv->v_scale;
  a.out = static_cast<uint16_t*>(out);
  a.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + w.partials);
  a.ld_table = ld_table;
  a.num_rows = num_rows;
  a.num_q_heads = num_q_heads;
  a.num_hgroups = p.hgroups;
  a.max_ctx = max_ctx;
  a.split_tok = p.split_tok;
  a.nsplit = p.nsplit;
  a.num_subpages = kv->num_pages * msa::kSubsPerPage;
  a.scale_log2 = sm_scale * msa::kLog2e;
  return a;
}

// Host checks of the fused step's arguments (everything but the workspace).
msa_status check_decode(const msa_batch* batch, const void* index_q, const void* index_k, const void* q,
                        int32_t num_q_heads, const msa_kv* kv, int32_t topk, const void* out,
                        const int32_t* sparse_table, const int32_t* ctx_lens, int32_t ld_s) {
  msa_status st = check_batch(batch, true);
  if (st != MSA_OK) return st;
  st = check_kv(kv);
  if (st != MSA_OK) return st;
  if (topk < 1 || num_q_heads < 1) return MSA_ERR_INVALID_ARG;
  if (topk > MSA_MAX_TOPK || num_q_heads > MSA_MAX_Q_HEADS) return MSA_ERR_UNSUPPORTED;
  if (batch->num_rows == 0) return MSA_OK;
  if (!index_q || !index_k || !q || !out || !sparse_table || !ctx_lens) return MSA_ERR_INVALID_ARG;
  if (ld_s < blocks_bound(batch) || ld_s < 1) return MSA_ERR_UNSUPPORTED;
  if (kv->num_pages != batch->num_pages) return MSA_ERR_INVALID_ARG;
  return MSA_OK;
}

msa_status launch_attn_and_merge(hipStream_t s, const MsaAttnArgs& a, const msa_kv* kv) {
  msa_status st = hip_status(msa_launch_attn(a, kv->kv_dtype, kv->scale_mode, s));
  if (st != MSA_OK) return st;
  return hip_status(msa_launch_merge(a, s));
}

}  // namespace

extern "C" {

msa_status msa_build_metadata(msa_stream_t stream, const msa_batch* batch) {
  msa_status st = check_batch(batch, true);
  if (st != MSA_OK) return st;
  if (batch->num_reqs == 0) return MSA_OK;
  return hip_status(msa_launch_meta(meta_args(batch), static_cast<hipStream_t>(stream)));
}

msa_status msa_index_score(msa_stream_t stream, const msa_batch* batch, const void* index_q, const void* index_k,
                           float* block_scores, int32_t ld_s) {
  return msa_index_score_ex(stream, batch, index_q, index_k, nullptr, block_scores, ld_s);
}

msa_status msa_index_score_ex(msa_stream_t stream, const msa_batch* batch, const void* index_q,
                              const void* index_k, const float* index_k_scale, float* block_scores, int32_t ld_s) {
  msa_status st = check_batch(batch, false);
  if (st != MSA_OK) return st;
  if (batch->num_rows == 0) return MSA_OK;
  if (!index_q || !index_k || !block_scores) return MSA_ERR_INVALID_ARG;
  if (ld_s < blocks_bound(batch) || ld_s < 1) return MSA_ERR_UNSUPPORTED;
  return launch_score(static_cast<hipStream_t>(stream), batch, index_q, index_k, index_k_scale, block_scores, ld_s,
                      false);
}

msa_status msa_topk_block_table(msa_stream_t stream, const msa_batch* batch, const float* block_scores,
                                int32_t ld_s, int32_t topk, int32_t* sparse_table, int32_t* ctx_lens,
                                int32_t* sel_blocks) {
  msa_status st = check_batch(batch, true);
  if (st != MSA_OK) return st;
  if (topk < 1) return MSA_ERR_INVALID_ARG;
  if (topk > MSA_MAX_TOPK) return MSA_ERR_UNSUPPORTED;
  if (batch->num_rows == 0) return MSA_OK;
  if (!block_scores || !sparse_table || !ctx_lens) return MSA_ERR_INVALID_ARG;
  if (ld_s < blocks_bound(batch) || ld_s < 1) return MSA_ERR_UNSUPPORTED;
  return launch_topk(static_cast<hipStream_t>(stream), batch, block_scores, ld_s, topk, sparse_table, ctx_lens,
                     sel_blocks);
}

msa_status msa_sparse_paged_attn(msa_stream_t stream, const void* q, int32_t num_rows, int32_t num_q_heads,
                                 const msa_kv* kv, const int32_t* sparse_table, int32_t ld_table,
                                 const int32_t* ctx_lens, int32_t max_ctx, float sm_scale, void* out,
                                 void* workspace, size_t workspace_bytes) {
  return msa_sparse_paged_attn_ex(stream, q, num_rows, num_q_heads, kv, sparse_table, ld_table, ctx_lens, max_ctx,
                                  sm_scale, nullptr, out, nullptr, workspace, workspace_bytes);
}

msa_status msa_sparse_paged_attn_ex(msa_stream_t stream, const void* q, int32_t num_rows, int32_t num_q_heads,
                                    const msa_kv* kv, const int32_t* sparse_table, int32_t ld_table,
                                    const int32_t* ctx_lens, int32_t max_ctx, float sm_scale, const float* sinks,
                                    void* out, float* lse, void* workspace, size_t workspace_bytes) {
  if (num_rows < 0 || max_ctx < 0 || ld_table < 0) return MSA_ERR_INVALID_ARG;
  if (num_q_heads < 1) return MSA_ERR_INVALID_ARG;
  if (num_q_heads > MSA_MAX_Q_HEADS || max_ctx > MSA_MAX_SEQ_LEN) return MSA_ERR_UNSUPPORTED;
  msa_status st = check_kv(kv);
  if (st != MSA_OK) return st;
  if (num_rows == 0) return MSA_OK;
  if (!q || !sparse_table || !ctx_lens || !out) return MSA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(ld_table) * kSub < max_ctx || ld_table < 1) return MSA_ERR_INVALID_ARG;
  const WsLayout w = ws_layout(num_rows, num_q_heads, max_ctx, 0);
  if (w.total > 0 && (!workspace || workspace_bytes < w.total)) return MSA_ERR_WORKSPACE;
  if (!attn_grid_fits(num_rows, num_q_heads, max_ctx)) return MSA_ERR_UNSUPPORTED;
  MsaAttnArgs a = attn_args(q, num_rows, num_q_heads, kv, ld_table, max_ctx, sm_scale, out, workspace);
  a.table_in = sparse_table;
  a.ctx_in = ctx_lens;
  a.sinks = sinks;
  a.lse_out = lse;
  return launch_attn_and_merge(static_cast<hipStream_t>(stream), a, kv);
}

msa_status msa_sparse_decode(msa_stream_t stream, const msa_batch* batch, const void* index_q, const void* index_k,
                             const void* q, int32_t num_q_heads, const msa_kv* kv, int32_t topk, float sm_scale,
                             void* out, int32_t* sparse_table, int32_t* ctx_lens, int32_t* sel_blocks,
                             float* block_scores, int32_t ld_s, void* workspace, size_t workspace_bytes) {
  return msa_sparse_decode_ex(stream, batch, index_q, index_k, nullptr, q, num_q_heads, kv, topk, sm_scale, nullptr,
                              out, nullptr, sparse_table, ctx_lens, sel_blocks, block_scores, ld_s, workspace,
                              workspace_bytes);
}

msa_status msa_sparse_decode_ex(msa_stream_t stream, const msa_batch* batch, const void* index_q, const void* index_k,
                                const float* index_k_scale, const void* q, int32_t num_q_heads, const msa_kv* kv,
                                int32_t topk, float sm_scale, const float* sinks, void* out, float* lse,
                                int32_t* sparse_table, int32_t* ctx_lens, int32_t* sel_blocks, float* block_scores,
                                int32_t ld_s, void* workspace, size_t workspace_bytes) {
  msa_status st = check_decode(batch, index_q, index_k, q, num_q_heads, kv, topk, out, sparse_table, ctx_lens, ld_s);
  if (st != MSA_OK) return st;
  if (batch->num_rows == 0) return batch->num_reqs ? msa_build_metadata(stream, batch) : MSA_OK;
  const int32_t max_ctx = kPage * topk;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (batch->num_rows >= kBlockMajorRows && batch->num_rows <= kBlockMajorMaxRows) {
    const int nbmax = blocks_bound(batch);
    const BmLayout bw = bm_layout(batch->num_rows, nbmax, num_q_heads, topk, block_scores ? 0 : ld_s);
    if (workspace && workspace_bytes >= bw.total) {
      // 1) metadata + index scores (unit and tile kernels), 2) top-k + table
      // + ctx + selection words, 3) rows per block (at most 16384 items),
      // 4) block-major attention, 5) merge of the block partials
      char* wsb = static_cast<char*>(workspace);
      float* scores = block_scores ? block_scores : reinterpret_cast<float*>(wsb + bw.scores);
      uint64_t* words = reinterpret_cast<uint64_t*>(wsb + bw.words);
      st = launch_score(s, batch, index_q, index_k, index_k_scale, scores, ld_s, true);
      if (st != MSA_OK) return st;
      MsaTopkArgs t = topk_args(batch, scores, ld_s, topk, sparse_table, ctx_lens, sel_blocks);
      t.row_words = words;
      t.row_words_ld = bm_words(nbmax);
      st = hip_status(msa_launch_topk(t, s));
      if (st != MSA_OK) return st;
      MsaAttnArgs a = attn_args(q, batch->num_rows, num_q_heads, kv, 8 * topk, max_ctx, sm_scale, out, workspace);
      a.partials = reinterpret_cast<float*>(wsb + bw.partials);
      a.nsplit = topk;  // one partial slot per selected block
      a.half_partials = 1;
      a.split_tok = kPage;
      a.ctx_in = ctx_lens;
      a.block_table = batch->block_table;
      a.ld_bt = batch->ld_bt;
      a.sinks = sinks;
      a.lse_out = lse;
      MsaBlockArgs bk;
      bk.row_words = words;
      bk.cu_q = batch->cu_seqlens_q;
      bk.seq_lens = batch->seq_lens;
      bk.row_words_ld = bm_words(nbmax);
      bk.nbmax = nbmax;
      bk.num_reqs = batch->num_reqs;
      bk.topk = topk;
      bk.len_cap = len_cap(batch);
      bk.counts = nullptr;
      if (nbmax >= 1 && static_cast<int64_t>(batch->num_reqs) * nbmax <= kBalancedItemsMax) {
        bk.counts = reinterpret_cast<int32_t*>(wsb + bw.counts);
        st = hip_status(msa_launch_block_count(bk, batch->num_rows, s));
        if (st != MSA_OK) return st;
      }
      int64_t wgs = static_cast<int64_t>(batch->num_reqs) * nbmax;
      if (wgs > 2LL * cu_count()) wgs = 2LL * cu_count();
      if (wgs < 1) wgs = 1;  // max_seq_len 0: no item, but a valid launch
      st = hip_status(msa_launch_attn_block(a, bk, kv->kv_dtype, kv->scale_mode, static_cast<int>(wgs), s));
      if (st != MSA_OK) return st;
      return hip_status(msa_launch_merge(a, s));
    }
  }
  const WsLayout w = ws_layout(batch->num_rows, num_q_heads, max_ctx, block_scores ? 0 : ld_s);
  if (w.total > 0 && (!workspace || workspace_bytes < w.total)) return MSA_ERR_WORKSPACE;
  if (!attn_grid_fits(batch->num_rows, num_q_heads, max_ctx)) return MSA_ERR_UNSUPPORTED;
  float* scores = block_scores ? block_scores : reinterpret_cast<float*>(static_cast<char*>(workspace) + w.scores);
  // 1) metadata + index scores, 2) per-row selection + attention, 3) split merge
  st = launch_score(s, batch, index_q, index_k, index_k_scale, scores, ld_s, true);
  if (st != MSA_OK) return st;
  MsaAttnArgs a = attn_args(q, batch->num_rows, num_q_heads, kv, 8 * topk, max_ctx, sm_scale, out, workspace);
  a.scores = scores;
  a.ld_s = ld_s;
  a.block_table = batch->block_table;
  a.ld_bt = batch->ld_bt;
  a.row_req = batch->row_req;
  a.row_pos = batch->row_pos;
  a.num_reqs = batch->num_reqs;
  a.topk = topk;
  a.table_out = sparse_table;
  a.ctx_out = ctx_lens;
  a.sel_out = sel_blocks;
  a.sinks = sinks;
  a.lse_out = lse;
  return launch_attn_and_merge(s, a, kv);
}

msa_status msa_sparse_decode_static(msa_stream_t stream, const msa_batch* batch, const void* index_q,
                                    const void* index_k, const float* index_k_scale, const void* q,
                                    int32_t num_q_heads, const msa_kv* kv, int32_t topk, float sm_scale,
                                    const float* sinks, void* out, float* lse, int32_t* sparse_table,
                                    int32_t* ctx_lens, int32_t* sel_blocks, float* block_scores, int32_t ld_s) {
  msa_status st = check_decode(batch, index_q, index_k, q, num_q_heads, kv, topk, out, sparse_table, ctx_lens, ld_s);
  if (st != MSA_OK) return st;
  if (batch->num_rows == 0)  // metadata only: no workspace
    return msa_sparse_decode_ex(stream, batch, index_q, index_k, index_k_scale, q, num_q_heads, kv, topk, sm_scale,
                                sinks, out, lse, sparse_table, ctx_lens, sel_blocks, block_scores, ld_s, nullptr, 0);
  // what the per-row path needs; a launch whose block-major workspace also
  // fits takes that path, exactly as msa_sparse_decode_ex given this size
  const size_t need = ws_layout(batch->num_rows, num_q_heads, kPage * topk, block_scores ? 0 : ld_s).total;
  if (need > static_cast<size_t>(MSA_STATIC_SCRATCH_BYTES)) return MSA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (static_scratch(&ws) != hipSuccess) return MSA_ERR_HIP;
  return msa_sparse_decode_ex(stream, batch, index_q, index_k, index_k_scale, q, num_q_heads, kv, topk, sm_scale,
                              sinks, out, lse, sparse_table, ctx_lens, sel_blocks, block_scores, ld_s, ws,
                              MSA_STATIC_SCRATCH_BYTES);
}

msa_status msa_cache_insert(msa_stream_t stream, int32_t num_tokens, const int32_t* slot_mapping, const void* k_new,
                            const void* v_new, const msa_kv* kv, const void* index_k_new, void* index_k) {
  return msa_cache_insert_ex(stream, num_tokens, slot_mapping, k_new, v_new, kv, index_k_new, index_k, nullptr);
}

msa_status msa_cache_insert_ex(msa_stream_t stream, int32_t num_tokens, const int32_t* slot_mapping,
                               const void* k_new, const void* v_new, const msa_kv* kv, const void* index_k_new,
                               void* index_k, float* index_k_scale) {
  msa_status st = check_kv(kv);
  if (st != MSA_OK) return st;
  if (num_tokens < 0) return MSA_ERR_INVALID_ARG;
  if (num_tokens == 0) return MSA_OK;
  if (!slot_mapping || !k_new || !v_new) return MSA_ERR_INVALID_ARG;
  if (index_k_new && !index_k) return MSA_ERR_INVALID_ARG;
  MsaInsertArgs a;
  a.slot_mapping = slot_mapping;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.index_k_new = static_cast<const uint16_t*>(index_k_new);
  // the caches (and per-token-head scales) are the call's outputs
  a.k_cache = const_cast<void*>(kv->k_cache);
  a.v_cache = const_cast<void*>(kv->v_cache);
  a.index_k = static_cast<uint16_t*>(index_k);
  a.k_scale = kv->k_scale;
  a.v_scale = kv->v_scale;
  a.k_scale_out = const_cast<float*>(kv->k_scale);
  a.v_scale_out = const_cast<float*>(kv->v_scale);
  a.index_scale_out = index_k_new ? index_k_scale : nullptr;
  a.num_tokens = num_tokens;
  a.num_pages = kv->num_pages;
  a.num_kv_heads = kv->num_kv_heads;
  a.kv_fp8 = kv->kv_dtype == MSA_KV_FP8_E4M3FN ? 1 : 0;
  a.scale_mode = kv->scale_mode;
  return hip_status(msa_launch_insert(a, static_cast<hipStream_t>(stream)));
}

size_t msa_workspace_bytes(int32_t num_rows, int32_t num_q_heads, int32_t max_ctx, int32_t ld_s) {
  if (num_rows < 0 || num_q_heads < 1 || max_ctx < 0 || ld_s < 0) return 0;
  return ws_layout(num_rows, num_q_heads, max_ctx, ld_s).total;
}

size_t msa_decode_workspace_bytes(int32_t num_rows, int32_t max_seq_len, int32_t num_q_heads, int32_t topk,
                                  int32_t ld_s) {
  if (num_rows < 0 || max_seq_len < 0 || num_q_heads < 1 || topk < 1 || ld_s < 0) return 0;
  const size_t per_row = ws_layout(num_rows, num_q_heads, kPage * topk, ld_s).total;
  if (num_rows < kBlockMajorRows || num_rows > kBlockMajorMaxRows) return per_row;
  const int nbmax = static_cast<int>(ceil_div(max_seq_len, kPage));
  const size_t bm = bm_layout(num_rows, nbmax, num_q_heads, topk, ld_s).total;
  return bm > per_row ? bm : per_row;
}

const char* msa_status_string(msa_status status) {
  switch (status) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
  }
  return "MSA_ERR_UNKNOWN";
}

int32_t msa_version(void) { return 200; }

}  // extern "C"

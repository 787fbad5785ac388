// Internal declarations of the top-k, attention and cache-insert kernels:
// their argument structs and launchers (host functions defined next to each
// kernel), which msa_api.hip calls. Not part of the public ABI.
#pragma once

#include "msa_internal.h"

namespace msa {

// Two floats -> two IEEE fp16 (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pk_f16(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}
// fp16 partial accumulators are scaled by 2^-e with |e| capped here: the
// sums they are folded into stay normal fp32 numbers, and accumulators up to
// 2^(kHalfExpRange+16) in magnitude stay finite.
constexpr int kHalfExpRange = 100;

}  // namespace msa

struct MsaTopkArgs {
  const float* scores;
  const int32_t* block_table;
  const int32_t* row_req;
  const int32_t* row_pos;
  int32_t* table;
  int32_t* ctx;
  int32_t* sel;        // may be null
  // Optional selection words (block-major attention): row n's kept blocks
  // as bits, block b at bit b%32 of word b/32, each 64-bit entry holding the
  // word in its low half and the number of kept blocks below the word in its
  // high half: row_words[n * row_words_ld + w] for every w < row_words_ld.
  // Null: not written.
  uint64_t* row_words;
  int32_t row_words_ld;
  int32_t ld_s;
  int32_t ld_bt;
  int32_t topk;
  int32_t num_rows;
  int32_t num_reqs;
};
hipError_t msa_launch_topk(const MsaTopkArgs& a, hipStream_t s);


// Attention over a page-16 table. Table mode: table_in / ctx_in give each
// row's sub-pages. Fused mode (scores != null): every workgroup selects its
// row's blocks from the block scores itself; the (split 0, head group 0)
// workgroup of a row writes table_out / ctx_out / sel_out.
struct MsaAttnArgs {
  const uint16_t* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* table_in;
  const int32_t* ctx_in;
  const float* scores;
  const int32_t* block_table;
  const int32_t* row_req;
  const int32_t* row_pos;
  int32_t* table_out;
  int32_t* ctx_out;
  int32_t* sel_out;    // may be null
  uint16_t* out;
  float* lse_out;      // [rows][Hq] natural-log LSE, or null
  const float* sinks;  // [Hq] per-head sink logits, or null
  // [rows][hgroups][nsplit] slots: m[16], l[16] fp32, then acc[16][128] fp16
  // scaled by a power of two folded into m and l
  float* partials;
  int32_t half_partials;  // block-major path: every row is merged from its slots (one slot too)
  int32_t ld_table;    // row stride of the table (8*topk in fused mode)
  int32_t ld_s;
  int32_t ld_bt;
  int32_t num_reqs;
  int32_t topk;
  int32_t num_rows;
  int32_t num_q_heads;
  int32_t num_hgroups;
  int32_t max_ctx;
  int32_t split_tok;   // tokens per workgroup, a power of two >= 64 (one sub-page per wave)
  int32_t nsplit;      // ceil(max_ctx / split_tok)
  int32_t num_subpages;
  float scale_log2;    // sm_scale * log2(e)
};
// New tokens into the paged caches (K / V planes, scales, index-K).
struct MsaInsertArgs {
  const int32_t* slot_mapping;   // [T] 128*page + offset; < 0: skipped
  const uint16_t* k_new;         // [T][Hkv][128] bf16
  const uint16_t* v_new;
  const uint16_t* index_k_new;   // [T][128] bf16, or null: the index cache is left alone
  void* k_cache;
  void* v_cache;
  uint16_t* index_k;
  const float* k_scale;          // scalar mode: [1], read
  const float* v_scale;
  float* k_scale_out;            // per-token-head mode: [8P][16][Hkv], written
  float* v_scale_out;
  float* index_scale_out;        // [P][128]: the index cache is fp8 and these scales are written; null: bf16
  int32_t num_tokens;
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t kv_fp8;
  int32_t scale_mode;
};
hipError_t msa_launch_insert(const MsaInsertArgs& a, hipStream_t s);

constexpr int kMaxSplitTokens = 8192;
hipError_t msa_launch_attn(const MsaAttnArgs& a, int kv_dtype, int scale_mode, hipStream_t s);
hipError_t msa_launch_merge(const MsaAttnArgs& a, hipStream_t s);
// Block-major attention (prefill-sized fused steps): a work item is a
// (request, block) and serves every row of the request that selected the
// block, found from the selection words written by the top-k kernel; items
// go to workgroups by grid stride, or balanced by cost when counts are given.
// Uses from MsaAttnArgs: q, caches and scales, block_table, ld_bt, out,
// lse_out, sinks, partials (nsplit = topk slots per row and head group),
// num_rows, num_q_heads, num_hgroups, num_subpages, scale_log2.
struct MsaBlockArgs {
  const uint64_t* row_words; // [N][row_words_ld] selection words written by the top-k kernel
  const int32_t* cu_q;       // [R+1] query-row prefix
  const int32_t* seq_lens;   // [R]
  int32_t row_words_ld;
  int32_t nbmax;             // blocks per request covered by the items
  int32_t num_reqs;
  int32_t topk;
  int32_t len_cap;
  int32_t* counts;           // [num_reqs][nbmax] rows per item (msa_block_count_kernel), or null:
                             // items by grid stride instead of entries balanced over the grid
};
hipError_t msa_launch_attn_block(const MsaAttnArgs& a, const MsaBlockArgs& b, int kv_dtype, int scale_mode,
                                 int num_wgs, hipStream_t s);
// Fills b.counts from the selection words (grid num_reqs x row_words_ld).
hipError_t msa_launch_block_count(const MsaBlockArgs& b, int num_rows, hipStream_t s);

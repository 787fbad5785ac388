// Fused top-k block selection, page-16 sparse block table and context length
// (vLLM PR #54682 page, 实现拆解 items 1 and 4: one pass selects each row's
// blocks and writes the page-16 table row and the context length; vLLM PR
// #47287 page, 实现拆解 item 3: the page-16 view of the page-128 cache, and
// 评论区精华: the zero padding must stay inside the allocated row).
//
// One 256-thread workgroup per query row: the row's scores are read once into
// LDS as keys, selected by select_row (msa_select.h), and every kept block j
// (ascending) is expanded to its 8 sub-pages 8*page + i. For block-major
// attention the kernel also writes the row's kept blocks as bit words.
#include "msa_select.h"

using namespace msa;

namespace {

// The row's keys live in dynamic LDS sized for the launch's block bound, so
// rows of a few hundred blocks leave room for many workgroups per compute
// unit (a static 8192-key array allowed four).
__global__ __launch_bounds__(kSelectThreads) void msa_topk_kernel(MsaTopkArgs a) {
  extern __shared__ uint32_t s_key[];  // [min(ld_s, ld_bt, kMaxBlocksPerRow)]
  __shared__ SelectLds sl;
  const int tid = threadIdx.x;
  const int n = blockIdx.x;
  const int r = clampi(a.row_req[n], 0, a.num_reqs - 1);
  const int v = a.row_pos[n] + 1;  // visible keys
  const int nb = clampi((v + kPage - 1) / kPage, 0, min(min(a.ld_s, a.ld_bt), kMaxBlocksPerRow));
  const float* srow = a.scores + static_cast<size_t>(n) * a.ld_s;
  const int32_t* bt = a.block_table + static_cast<size_t>(r) * a.ld_bt;
  int32_t* trow = a.table + static_cast<size_t>(n) * (8 * a.topk);
  int32_t* selrow = a.sel ? a.sel + static_cast<size_t>(n) * a.topk : nullptr;

  __shared__ uint32_t s_bits[kMaxBlocksPerRow / 32];  // kept blocks as bits, for the selection words
  if (a.row_words && tid < kMaxBlocksPerRow / 32) s_bits[tid] = 0u;
  for (int e = tid; e < nb; e += kSelectThreads) s_key[e] = order_key(srow[e]);
  __syncthreads();

  int ctx = 0;
  const int kk = select_row(s_key, nb, a.topk, v, sl, [&](int pos, int e) {
    const int32_t sub0 = 8 * bt[e];
#pragma unroll
    for (int i = 0; i < 8; ++i) trow[8 * pos + i] = sub0 + i;
    if (selrow) selrow[pos] = e;
    if (a.row_words) atomicOr(&s_bits[e >> 5], 1u << (e & 31));
  }, &ctx, [] {});

  if (a.row_words) {  // every word of the row, with the kept count below it
    __syncthreads();
    for (int w = tid; w < a.row_words_ld; w += kSelectThreads) {
      uint32_t below = 0, bits = 0;
      for (int u = 0; u < min(w, kMaxBlocksPerRow / 32); ++u) below += __popc(s_bits[u]);
      if (w < kMaxBlocksPerRow / 32) bits = s_bits[w];
      a.row_words[static_cast<size_t>(n) * a.row_words_ld + w] = (static_cast<uint64_t>(below) << 32) | bits;
    }
  }

  // zero tail of the table row, -1 tail of the selection, never past 8*topk
  for (int m = 8 * kk + tid; m < 8 * a.topk; m += kSelectThreads) trow[m] = 0;
  if (selrow)
    for (int m = kk + tid; m < a.topk; m += kSelectThreads) selrow[m] = -1;
  if (tid == 0) a.ctx[n] = ctx;
}

}  // namespace

hipError_t msa_launch_topk(const MsaTopkArgs& a, hipStream_t s) {
  const int nbmax = a.ld_s < a.ld_bt ? a.ld_s : a.ld_bt;
  const size_t key_bytes = sizeof(uint32_t) * static_cast<size_t>(nbmax < kMaxBlocksPerRow ? nbmax : kMaxBlocksPerRow);
  hipLaunchKernelGGL(msa_topk_kernel, dim3(a.num_rows), dim3(kSelectThreads), key_bytes, s, a);
  return hipGetLastError();
}

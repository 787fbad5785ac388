// Fused top-k block selection, page-16 sparse block table and context length
// (vLLM PR #54682 page, 实现拆解 items 1 and 4: one pass selects each row's
// blocks and writes the page-16 table row and the context length; vLLM PR
// #47287 page, 实现拆解 item 3: the page-16 view of the page-128 cache, and
// 评论区精华: the zero padding must stay inside the allocated row).
//
// One wave per query row, four rows per 256-thread workgroup: the row's
// keys and block-table entries sit in registers (lane l holds blocks
// l + 64*j), the wave selects alone (wave_select: the MSB-first radix select
// in the wave's own LDS histograms, no workgroup barrier), and every lane
// holding a kept block writes that block's 8 table entries at its rank,
// counted from the keep ballots of the 64-block chunks below it. For
// block-major attention the kernel also writes the row's kept blocks as bit
// words.
#include "msa_select.h"

using namespace msa;

namespace {

template <int KR>
__global__ __launch_bounds__(kSelectThreads) void msa_topk_kernel(MsaTopkArgs a) {
  __shared__ __attribute__((aligned(16))) int s_hist[4][kWaveRadixPasses][256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int n = static_cast<int>(blockIdx.x) * 4 + wave;
  if (n >= a.num_rows) return;
  const int nbmax = min(min(a.ld_s, a.ld_bt), kMaxBlocksPerRow);
  const float* srow = a.scores + static_cast<size_t>(n) * a.ld_s;
  // keys and the row's request first (indices clamped: every load issues)
  WaveKeys<KR> wk;
  float kraw[KR];
#pragma unroll
  for (int j = 0; j < KR; ++j) kraw[j] = srow[min(lane + 64 * j, max(nbmax, 1) - 1)];
  const int r = clampi(a.row_req[n], 0, a.num_reqs - 1);
  const int v = a.row_pos[n] + 1;  // visible keys
  wave_clear_hist(s_hist[wave]);
  const int nb = clampi((v + kPage - 1) / kPage, 0, nbmax);
  const int32_t* bt = a.block_table + static_cast<size_t>(r) * a.ld_bt;
  int pg[KR];
#pragma unroll
  for (int j = 0; j < KR; ++j) pg[j] = bt[min(lane + 64 * j, max(nb, 1) - 1)];
#pragma unroll
  for (int j = 0; j < KR; ++j) wk.k[j] = order_key(kraw[j]);
  auto tail_key = [&](int e) { return order_key(srow[e]); };
  wave_lds_order();  // histograms cleared
  const WaveSelection ws = wave_select(wk, nb, a.topk, s_hist[wave], tail_key);

  int32_t* trow = a.table + static_cast<size_t>(n) * (8 * a.topk);
  int32_t* selrow = a.sel ? a.sel + static_cast<size_t>(n) * a.topk : nullptr;
  uint64_t* wrow = a.row_words ? a.row_words + static_cast<size_t>(n) * a.row_words_ld : nullptr;
  const uint64_t lt = (1ull << lane) - 1ull;
  int carry = 0, carry_eq = 0;
  bool last_kept = false;
  auto keep_of = [&](bool valid, uint32_t k) {
    if (!ws.partial) return valid;
    if (ws.all_eq_kept) return valid && k >= ws.T;
    // keys equal to the threshold are kept in ascending block order
    const bool eq = valid && k == ws.T;
    const uint64_t em = __ballot(eq);
    const int rank_eq = carry_eq + __popcll(em & lt);
    carry_eq += __popcll(em);
    return valid && (k > ws.T || (eq && rank_eq < ws.need));
  };
  // one 64-block chunk: the kept blocks' table entries and selection at their
  // ranks, and the chunk's two selection words
  auto chunk = [&](int base, uint32_t k, int page) {
    const bool keep = keep_of(base + lane < nb, k);
    const uint64_t km = __ballot(keep);
    if (keep) {
      const int rank = carry + __popcll(km & lt);
      const int32_t sub0 = 8 * page;
#pragma unroll
      for (int i = 0; i < 8; ++i) trow[8 * rank + i] = sub0 + i;
      if (selrow) selrow[rank] = base + lane;
    }
    if (nb - 1 - base >= 0 && nb - 1 - base < 64) last_kept = (km >> (nb - 1 - base)) & 1ull;
    if (wrow && lane < 2 && (base >> 5) + lane < a.row_words_ld) {
      const uint32_t lo = static_cast<uint32_t>(km);
      const uint32_t bits = lane ? static_cast<uint32_t>(km >> 32) : lo;
      const uint32_t below = static_cast<uint32_t>(carry) + (lane ? static_cast<uint32_t>(__popc(lo)) : 0u);
      wrow[(base >> 5) + lane] = (static_cast<uint64_t>(below) << 32) | bits;
    }
    carry += __popcll(km);
  };
#pragma unroll
  for (int j = 0; j < KR; ++j)
    if (64 * j < nb) chunk(64 * j, wk.k[j], pg[j]);
  for (int base = 64 * KR; base < nb; base += 64) {
    const int e = min(base + lane, nb - 1);
    chunk(base, tail_key(e), bt[e]);
  }
  if (wrow)  // words past the row's blocks: no bits, every kept block below
    for (int w = 2 * ((nb + 63) >> 6) + lane; w < a.row_words_ld; w += 64)
      wrow[w] = static_cast<uint64_t>(ws.kk) << 32;
  // zero tail of the table row, -1 tail of the selection, never past 8*topk
  for (int m = 8 * ws.kk + lane; m < 8 * a.topk; m += 64) trow[m] = 0;
  if (selrow)
    for (int m = ws.kk + lane; m < a.topk; m += 64) selrow[m] = -1;
  if (lane == 0) a.ctx[n] = kPage * ws.kk - (last_kept ? kPage * nb - v : 0);
}

}  // namespace

hipError_t msa_launch_topk(const MsaTopkArgs& a, hipStream_t s) {
  const int nbmax = a.ld_s < a.ld_bt ? a.ld_s : a.ld_bt;
  const dim3 grid(static_cast<unsigned>((a.num_rows + 3) / 4));
  if (nbmax <= 256)
    hipLaunchKernelGGL(msa_topk_kernel<4>, grid, dim3(kSelectThreads), 0, s, a);
  else
    hipLaunchKernelGGL(msa_topk_kernel<16>, grid, dim3(kSelectThreads), 0, s, a);
  return hipGetLastError();
}

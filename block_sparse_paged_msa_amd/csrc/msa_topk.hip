// Fused top-k block selection, page-16 sparse block table and context length
// (vLLM PR #54682 page, 实现拆解 items 1 and 4: one pass selects each row's
// blocks and writes the page-16 table row and the context length; vLLM PR
// #47287 page, 实现拆解 item 3: the page-16 view of the page-128 cache, and
// 评论区精华: the zero padding must stay inside the allocated row).
//
// One 256-thread workgroup per query row. The K'-th largest block score is
// found by an MSB-first radix select over order-preserving 32-bit keys (4
// passes of 8 bits, histograms in LDS). Ties at the threshold are resolved by
// ascending block id with a block-wide prefix count, and the kept blocks are
// compacted in ascending id order with a second prefix count, which is also
// the order the table is written in.
#include "msa_internal.h"

using namespace msa;

namespace {

constexpr int kTopkThreads = 256;

// Larger float -> larger unsigned key; -0.0 maps to the key of +0.0.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__global__ __launch_bounds__(kTopkThreads) void msa_topk_kernel(MsaTopkArgs a) {
  __shared__ int s_hist[256];
  __shared__ int s_scan[4];
  __shared__ int s_digit, s_need;
  __shared__ int s_ctx[4];
  const int tid = threadIdx.x;
  const int n = blockIdx.x;
  const int r = clampi(a.row_req[n], 0, a.num_reqs - 1);
  const int v = a.row_pos[n] + 1;                              // visible keys
  const int nb = clampi((v + kPage - 1) / kPage, 0, min(a.ld_s, a.ld_bt));   // eligible blocks
  const int kk = min(a.topk, nb);
  const float* srow = a.scores + static_cast<size_t>(n) * a.ld_s;
  const int32_t* bt = a.block_table + static_cast<size_t>(r) * a.ld_bt;
  int32_t* trow = a.table + static_cast<size_t>(n) * (8 * a.topk);

  // ---- threshold key T and how many blocks equal to T are kept ----
  uint32_t T = 0;
  int need = 0;
  const bool partial = kk < nb;
  if (partial) {
    uint32_t prefix = 0;
    need = kk;
    for (int shift = 24; shift >= 0; shift -= 8) {
      s_hist[tid] = 0;
      __syncthreads();
      for (int e = tid; e < nb; e += kTopkThreads) {
        const uint32_t k = order_key(srow[e]);
        const bool match = (shift == 24) || ((k >> (shift + 8)) == (prefix >> (shift + 8)));
        if (match) atomicAdd(&s_hist[(k >> shift) & 255u], 1);
      }
      __syncthreads();
      const int c = s_hist[255 - tid];                 // digits in descending order
      int tot;
      const int excl = block256_exclusive_scan(c, s_scan, &tot);
      if (excl < need && need <= excl + c) {
        s_digit = 255 - tid;
        s_need = need - excl;
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(s_digit) << shift;
      need = s_need;
      __syncthreads();
    }
    T = prefix;
  }

  // ---- keep: key > T, or key == T among the first `need` by id; compact ----
  int carry_eq = 0, carry_sel = 0, ctx = 0;
  for (int base = 0; base < nb; base += kTopkThreads) {
    const int e = base + tid;
    const bool valid = e < nb;
    const uint32_t k = valid ? order_key(srow[e]) : 0u;
    const int eq = (partial && valid && k == T) ? 1 : 0;
    int tot_eq;
    const int rank_eq = carry_eq + block256_exclusive_scan(eq, s_scan, &tot_eq);
    const int keep = valid && (!partial || k > T || (eq && rank_eq < need)) ? 1 : 0;
    int tot_sel;
    const int pos = carry_sel + block256_exclusive_scan(keep, s_scan, &tot_sel);
    if (keep) {
      const int32_t sub0 = 8 * bt[e];
#pragma unroll
      for (int i = 0; i < 8; ++i) trow[8 * pos + i] = sub0 + i;
      if (a.sel) a.sel[static_cast<size_t>(n) * a.topk + pos] = e;
      ctx += min(kPage, v - kPage * e);
    }
    carry_eq += tot_eq;
    carry_sel += tot_sel;
  }

  // zero tail of the table row, -1 tail of the selection, never past 8*topk
  for (int m = 8 * kk + tid; m < 8 * a.topk; m += kTopkThreads) trow[m] = 0;
  if (a.sel)
    for (int m = kk + tid; m < a.topk; m += kTopkThreads) a.sel[static_cast<size_t>(n) * a.topk + m] = -1;

  // context length = sum of the kept blocks' visible tokens
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ctx += __shfl_xor(ctx, o);
  if ((tid & 63) == 0) s_ctx[tid >> 6] = ctx;
  __syncthreads();
  if (tid == 0) a.ctx[n] = s_ctx[0] + s_ctx[1] + s_ctx[2] + s_ctx[3];
}

}  // namespace

hipError_t msa_launch_topk(const MsaTopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(msa_topk_kernel, dim3(a.num_rows), dim3(kTopkThreads), 0, s, a);
  return hipGetLastError();
}

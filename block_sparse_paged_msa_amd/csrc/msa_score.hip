// Index scores pooled per 128-token block (vLLM PR #54682 page, 功能与动机 and
// 实现拆解 item 1: the per-row decode scorer with work mapped to each request's
// real block count, index-K tiles shared by all query rows of a request).
//
// Work unit = (request r, page j, group of up to 64 query rows of r). Units are
// numbered by the device prefix cu_units, so a persistent grid covers exactly
// the real pages of the batch (no per-request fixed grid). One wave owns one
// unit: it streams the 32 KiB index-K page into registers once (the B operand
// of v_mfma_f32_16x16x32_bf16, token = column) and multiplies it with every
// 16-row tile of the group's index queries (the A operand), so the page is
// shared by all of the request's rows that fall in the group. The max over the
// block's visible tokens is taken on the MFMA output, per row.
#include "msa_internal.h"

using namespace msa;

namespace {

constexpr int kScoreThreads = 256;
constexpr int kWavesPerWg = kScoreThreads / 64;

__device__ __forceinline__ void score_unit(const MsaScoreArgs& a, int u, int lane) {
  // request of this unit: last r with cu_units[r] <= u
  int lo = 0, hi = a.num_reqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_units[mid] <= u) lo = mid; else hi = mid;
  }
  const int r = lo;
  const int q0 = a.cu_q[r];
  const int ql = a.cu_q[r + 1] - q0;
  const int L = a.cu_k[r + 1] - a.cu_k[r];
  const int ngroups = (ql + kRowsPerUnit - 1) / kRowsPerUnit;
  const int local = u - a.cu_units[r];
  const int j = local / ngroups;                 // page (block) index inside the request
  const int g0 = (local - j * ngroups) * kRowsPerUnit;
  const int nrows = min(kRowsPerUnit, ql - g0);
  const int row0 = q0 + g0;                      // first query row of the group
  const int pos0 = L - ql + g0;                  // its absolute position
  const int nb_r = (L + kPage - 1) / kPage;

  const int page = clampi(a.block_table[static_cast<size_t>(r) * a.ld_bt + j], 0, a.num_pages - 1);
  const uint16_t* kp = a.index_k + static_cast<size_t>(page) * (kPage * kDim);

  // B operand: column = token tt*16 + lane%16, K entries = dims kc*32 + 8*(lane/16) .. +7
  bf16x8 kb[8][4];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt)
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
      kb[tt][kc] = *reinterpret_cast<const bf16x8*>(
          kp + (tt * 16 + (lane & 15)) * kDim + kc * 32 + (lane >> 4) * 8);

  const int t_base = j * kPage + (lane & 15);
  for (int mt = 0; mt * 16 < nrows; ++mt) {
    const int mrow = mt * 16 + (lane & 15);
    bf16x8 qa[4];
    if (mrow < nrows && row0 + mrow < a.num_rows) {
      const uint16_t* qp = a.index_q + static_cast<size_t>(row0 + mrow) * kDim + (lane >> 4) * 8;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) qa[kc] = *reinterpret_cast<const bf16x8*>(qp + kc * 32);
    } else {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) qa[kc] = bf16x8{};
    }
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) acc = mfma_16x16x32(qa[kc], kb[tt][kc], acc);
      const int t = t_base + tt * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mt * 16 + 4 * (lane >> 4) + i;
        const bool visible = (m < nrows) && (t <= pos0 + m);
        mx[i] = fmaxf(mx[i], visible ? acc[i] : -INFINITY);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) mx[i] = max16(mx[i]);
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mt * 16 + 4 * (lane >> 4) + i;
        if (m < nrows && row0 + m < a.num_rows)
          a.scores[static_cast<size_t>(row0 + m) * a.ld_s + j] = mx[i];
      }
    }
  }

  // the unit of the request's last page also writes the -inf tail of its rows
  if (j == nb_r - 1) {
    const int width = a.ld_s - nb_r;
    for (int idx = lane; idx < nrows * width; idx += 64) {
      const int m = idx / width;
      const int b = nb_r + (idx - m * width);
      if (row0 + m < a.num_rows) a.scores[static_cast<size_t>(row0 + m) * a.ld_s + b] = -INFINITY;
    }
  }
}

__global__ __launch_bounds__(kScoreThreads) void msa_score_kernel(MsaScoreArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int total = a.cu_units[a.num_reqs];
  const int nwaves = gridDim.x * kWavesPerWg;
  for (int u = blockIdx.x * kWavesPerWg + wave; u < total; u += nwaves) score_unit(a, u, lane);
}

}  // namespace

hipError_t msa_launch_score(const MsaScoreArgs& a, int num_wgs, hipStream_t s) {
  hipLaunchKernelGGL(msa_score_kernel, dim3(num_wgs), dim3(kScoreThreads), 0, s, a);
  return hipGetLastError();
}

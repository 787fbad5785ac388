// Device-side batch metadata (vLLM PR #56170 page, 实现拆解 items 1-3 and
// 关键源码片段): cumulative query / KV lengths start with a zero written on the
// device, each query row gets its request id and absolute position
// (context_len + i, context_len = seq_len - query_len), all without a host
// round trip.
#include "msa_internal.h"

using namespace msa;

namespace {

constexpr int kMetaThreads = 1024;
constexpr int kMetaWaves = kMetaThreads / 64;

__global__ __launch_bounds__(kMetaThreads) void msa_meta_kernel(MsaMetaArgs a) {
  __shared__ int s_cuq[kMaxReqs + 1];
  __shared__ int s_tot[kMetaWaves][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool writer = blockIdx.x == 0;
  const int R = a.num_reqs;

  if (tid == 0) {
    s_cuq[0] = 0;
    if (writer) {
      a.cu_q[0] = 0;
      a.cu_k[0] = 0;
      a.cu_blocks[0] = 0;
      a.cu_units[0] = 0;
    }
  }
  // Running sums of (query rows, KV tokens, 128-token blocks, score units),
  // 1024 requests at a time: a wave-level inclusive scan, then the wave totals.
  int cq = 0, ck = 0, cb = 0, cu = 0;
  for (int base = 0; base < R; base += kMetaThreads) {
    const int r = base + tid;
    int L = 0, ql = 0;
    if (r < R) {
      L = clampi(a.seq_lens[r], 0, a.len_cap);
      ql = clampi(a.query_lens[r], 0, L);
    }
    const int nb = (L + kPage - 1) / kPage;
    int x[4] = {ql, L, nb, nb * ((ql + kRowsPerUnit - 1) / kRowsPerUnit)};
#pragma unroll
    for (int c = 0; c < 4; ++c) x[c] = wave_inclusive_scan(x[c]);
    if (lane == 63) {
#pragma unroll
      for (int c = 0; c < 4; ++c) s_tot[wave][c] = x[c];
    }
    __syncthreads();
    int pre[4] = {cq, ck, cb, cu}, tot[4] = {0, 0, 0, 0};
    for (int w = 0; w < kMetaWaves; ++w) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pre[c] += (w < wave) ? s_tot[w][c] : 0;
        tot[c] += s_tot[w][c];
      }
    }
    __syncthreads();
    if (r < R) {
      s_cuq[r + 1] = pre[0] + x[0];
      if (writer) {
        a.cu_q[r + 1] = pre[0] + x[0];
        a.cu_k[r + 1] = pre[1] + x[1];
        a.cu_blocks[r + 1] = pre[2] + x[2];
        a.cu_units[r + 1] = pre[3] + x[3];
      }
    }
    cq += tot[0];
    ck += tot[1];
    cb += tot[2];
    cu += tot[3];
  }
  __syncthreads();

  // Each query row: its request is the last r with cu_q[r] <= n (empty
  // requests share a boundary and are skipped by taking the last one).
  for (int n = blockIdx.x * kMetaThreads + tid; n < a.num_rows; n += gridDim.x * kMetaThreads) {
    int lo = 0, hi = R;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_cuq[mid] <= n) lo = mid; else hi = mid;
    }
    const int L = clampi(a.seq_lens[lo], 0, a.len_cap);
    const int ql = s_cuq[lo + 1] - s_cuq[lo];
    a.row_req[n] = lo;
    a.row_pos[n] = clampi(L - ql + (n - s_cuq[lo]), -1, L - 1);
  }
}

}  // namespace

hipError_t msa_launch_meta(const MsaMetaArgs& a, hipStream_t s) {
  int64_t g = (static_cast<int64_t>(a.num_rows) + kMetaThreads - 1) / kMetaThreads;
  int grid = static_cast<int>(g < 1 ? 1 : (g > 64 ? 64 : g));
  hipLaunchKernelGGL(msa_meta_kernel, dim3(grid), dim3(kMetaThreads), 0, s, a);
  return hipGetLastError();
}


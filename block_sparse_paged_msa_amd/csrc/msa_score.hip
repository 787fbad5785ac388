// Index scores pooled per 128-token block (vLLM PR #54682 page, 功能与动机 and
// 实现拆解 item 1: the per-row decode scorer with work mapped to each request's
// real block count, index-K tiles shared by all query rows of a request).
//
// Work unit = (request r, page j, group of up to 64 query rows of r). Every
// workgroup first forms the running sums of query rows and units over the
// requests in LDS (from seq_lens / query_lens, one coalesced read), so a unit
// finds its request with an LDS binary search and the persistent grid covers
// exactly the real pages of the batch. In the fused decode step workgroup 0
// also writes the batch metadata (cu_seqlens_q/k, cu_blocks, cu_units, row
// request ids and positions: vLLM PR #56170 page, 实现拆解 items 1-3) so that
// no separate metadata launch is needed.
//
// One wave owns one unit: it streams the 32 KiB index-K page into registers
// once, in 1 KiB fully coalesced runs thanks to the shuffled tile layout (the
// B operand of v_mfma_f32_16x16x32_bf16, token = column) and
// multiplies it with every 16-row tile of the group's index queries (the A
// operand), so the page is shared by all of the request's rows in the group.
// The max over the block's visible tokens is taken on the MFMA output, per row.
#include "msa_internal.h"

using namespace msa;

namespace {

constexpr int kScoreThreads = 256;
constexpr int kWavesPerWg = kScoreThreads / 64;

__device__ __forceinline__ void score_unit(const MsaScoreArgs& a, const int* s_units, const int* s_cuq, int u,
                                           int lane) {
  int lo = 0, hi = a.num_reqs;  // request of this unit: last r with cu_units[r] <= u
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_units[mid] <= u) lo = mid; else hi = mid;
  }
  const int r = lo;
  const int q0 = s_cuq[r];
  const int ql = s_cuq[r + 1] - q0;
  const int ngroups = (ql + kRowsPerUnit - 1) / kRowsPerUnit;
  const int local = u - s_units[r];
  const int j = local / ngroups;                 // page (block) index inside the request
  const int g0 = (local - j * ngroups) * kRowsPerUnit;
  const int nrows = min(kRowsPerUnit, ql - g0);
  const int row0 = q0 + g0;                      // first query row of the group
  const int L = clampi(a.seq_lens[r], 0, a.len_cap);
  const int page = clampi(a.block_table[static_cast<size_t>(r) * a.ld_bt + j], 0, a.num_pages - 1);
  const int pos0 = L - ql + g0;                  // absolute position of the group's first row
  const int nb_r = (L + kPage - 1) / kPage;
  const uint16_t* kp = a.index_k + static_cast<size_t>(page) * (kPage * kDim);

  // B operand: column = token tt*16 + lane%16, K entries = dims kc*32 + 8*(lane/16) .. +7.
  // A page is 8 shuffled 16-token tiles [4][4][16][8], so each (tt, kc) operand
  // is one contiguous 1 KiB run read by the 64 lanes in order.
  bf16x8 kb[8][4];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt)
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
      kb[tt][kc] = *reinterpret_cast<const bf16x8*>(kp + tt * (kSub * kDim) + (kc * 64 + lane) * 8);

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
  extern __shared__ int s_dyn[];            // [R+1] unit prefix, [R+1] row prefix
  __shared__ int s_tot[kWavesPerWg][4];
  int* s_units = s_dyn;
  int* s_cuq = s_dyn + a.num_reqs + 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int R = a.num_reqs;
  const bool writer = a.write_meta && blockIdx.x == 0;

  if (tid == 0) {
    s_units[0] = 0;
    s_cuq[0] = 0;
    if (writer) {
      a.cu_q[0] = 0;
      a.cu_k[0] = 0;
      a.cu_blocks[0] = 0;
      a.cu_units[0] = 0;
    }
  }
  // running sums of (query rows, KV tokens, blocks, score units) over requests
  int carry[4] = {0, 0, 0, 0};
  for (int base = 0; base < R; base += kScoreThreads) {
    const int r = base + tid;
    int L = 0, ql = 0;
    if (r < R) {
      L = clampi(a.seq_lens[r], 0, a.len_cap);
      ql = clampi(a.query_lens[r], 0, L);
    }
    const int nb = (L + kPage - 1) / kPage;
    int x[4] = {ql, L, nb, nb * ((ql + kRowsPerUnit - 1) / kRowsPerUnit)};
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int y = __shfl_up(x[c], o);
        if (lane >= o) x[c] += y;
      }
    }
    if (lane == 63) {
#pragma unroll
      for (int c = 0; c < 4; ++c) s_tot[wave][c] = x[c];
    }
    __syncthreads();
    int pre[4], tot[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      pre[c] = carry[c];
      tot[c] = 0;
    }
#pragma unroll
    for (int w = 0; w < kWavesPerWg; ++w)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pre[c] += (w < wave) ? s_tot[w][c] : 0;
        tot[c] += s_tot[w][c];
      }
    __syncthreads();
    if (r < R) {
      s_cuq[r + 1] = pre[0] + x[0];
      s_units[r + 1] = pre[3] + x[3];
      if (writer) {
        a.cu_q[r + 1] = pre[0] + x[0];
        a.cu_k[r + 1] = pre[1] + x[1];
        a.cu_blocks[r + 1] = pre[2] + x[2];
        a.cu_units[r + 1] = pre[3] + x[3];
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) carry[c] += tot[c];
  }
  __syncthreads();

  if (writer) {  // per-row request id and absolute position
    for (int n = tid; n < a.num_rows; n += kScoreThreads) {
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

  const int total = s_units[R];
  const int nwaves = gridDim.x * kWavesPerWg;
  for (int u = blockIdx.x * kWavesPerWg + wave; u < total; u += nwaves) score_unit(a, s_units, s_cuq, u, lane);
}

}  // namespace

hipError_t msa_launch_score(const MsaScoreArgs& a, int num_wgs, hipStream_t s) {
  const size_t lds = sizeof(int) * 2 * static_cast<size_t>(a.num_reqs + 1);
  hipLaunchKernelGGL(msa_score_kernel, dim3(num_wgs), dim3(kScoreThreads), lds, s, a);
  return hipGetLastError();
}

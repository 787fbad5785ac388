// Index scores pooled per 128-token block for requests with many query rows
// (prefill chunks): an MFMA tile over (512 query rows of one request) x (a
// run of index-K pages), the rows' index queries kept in registers and the
// pages streamed once per workgroup through LDS (vLLM PR #54682 page, 实现拆解
// item 1: index-K tiles shared by the request's rows; the prefill-shaped
// scorer is the prefill counterpart named with PR #53448 among 相关 PRs).
//
// Workgroup = eight waves (one per compute unit), wave w owning rows
// 64w .. 64w+63 of a 512-row block as four 16-row A operands (64 registers).
// Each page (32 KiB of bf16, or 16 KiB of e4m3fn codes plus 128 scales) is
// copied global -> registers -> LDS by all 512 threads (64 bytes each),
// double-buffered: the next page is requested when the current one starts,
// so its loads have a whole page of products to arrive. Per page and wave:
//   S^T[token][row] = K_page (128x128) . Q^T (128x64)   128 x v_mfma_f32_16x16x32_bf16
// and each row keeps the max over the page's tokens it can see (t <= pos);
// in the S^T layout a lane's four outputs are four tokens of one row, so the
// max is mostly taken inside the lane, with one cross-lane merge per page.
// Pages past every row's position get -inf without being read; the work
// item holding a request's last page also writes the -inf tail up to ld_s.
// Only requests with more than 64 query rows are taken here; the unit kernel
// (msa_score.hip) skips them in the same launch pair.
#include <type_traits>

#include "msa_internal.h"

using namespace msa;

namespace {

constexpr int kTileWaves = 8;
constexpr int kTileThreads = 64 * kTileWaves;
constexpr int kWaveRows = 64;                  // per wave: four 16-row MFMA tiles
constexpr int kTileRows = kWaveRows * kTileWaves;  // query rows per workgroup
constexpr int kRunPages = 8;                   // pages per work item (or twice as many, below)

template <int IDX_FP8>
struct TileShared {
  static constexpr int kPageBytes = kPage * kDim * (IDX_FP8 ? 1 : 2);
  __attribute__((aligned(16))) uint8_t page[2][kPageBytes];
  float scale[2][kPage];
};

// Staging registers of one page: 16-byte pieces tid + 512*i.
template <int IDX_FP8>
struct PageStage {
  static constexpr int kPieces = TileShared<IDX_FP8>::kPageBytes / 16 / kTileThreads;  // 4 or 2
  u32x4 v[kPieces];
  float sc;

  __device__ __forceinline__ void load(const MsaScoreArgs& a, int page, int tid) {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.index_k) +
                                                      static_cast<size_t>(page) * TileShared<IDX_FP8>::kPageBytes);
#pragma unroll
    for (int i = 0; i < kPieces; ++i) v[i] = __builtin_nontemporal_load(src + tid + kTileThreads * i);
    if constexpr (IDX_FP8 != 0) sc = a.index_scale[static_cast<size_t>(page) * kPage + (tid & (kPage - 1))];
  }
  __device__ __forceinline__ void store(TileShared<IDX_FP8>& sh, int buf, int tid) const {
    u32x4* dst = reinterpret_cast<u32x4*>(sh.page[buf]);
#pragma unroll
    for (int i = 0; i < kPieces; ++i) dst[tid + kTileThreads * i] = v[i];
    if constexpr (IDX_FP8 != 0) {
      if (tid < kPage) sh.scale[buf][tid] = sc;
    }
  }
};

// Exclusive prefix sum over the workgroup's threads (and the total).
__device__ __forceinline__ int tile_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_inclusive_scan(v);
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTileWaves; ++w) {
    const int t = scratch[w];
    base += (w < wave) ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// B operand (tt, kc) of a page in LDS: token tt*16 + lane%16, dims
// kc*32 + 8*(lane/16) .. +7 (the tile layout is the operand order).
template <int IDX_FP8>
__device__ __forceinline__ bf16x8 lds_operand(const TileShared<IDX_FP8>& sh, int buf, int tt, int kc, int lane) {
  const int piece = (tt * 4 + kc) * 64 + lane;
  if constexpr (IDX_FP8 != 0) {
    const u32x2 w = reinterpret_cast<const u32x2*>(sh.page[buf])[piece];
    const u32x2 lo = fp8x4_to_bf16x4(w.x), hi = fp8x4_to_bf16x4(w.y);
    return __builtin_bit_cast(bf16x8, (u32x4{lo.x, lo.y, hi.x, hi.y}));
  } else {
    return reinterpret_cast<const bf16x8*>(sh.page[buf])[piece];
  }
}

template <int IDX_FP8>
__global__ __launch_bounds__(kTileThreads, 1) void msa_score_tile_kernel(MsaScoreArgs a) {
  extern __shared__ int s_dyn[];  // [R+1] row prefix, [R+1] work-item prefix for runs of 8 and of 16 pages
  __shared__ TileShared<IDX_FP8> sh;
  __shared__ int s_scan[kTileWaves];
  int* s_cuq = s_dyn;
  int* s_items = s_dyn + a.num_reqs + 1;
  int* s_items2 = s_dyn + 2 * (a.num_reqs + 1);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int R = a.num_reqs;

  // running sums over the requests of query rows and of this kernel's work
  // items (requests with more than 64 rows: row blocks x page runs)
  if (tid == 0) {
    s_cuq[0] = 0;
    s_items[0] = 0;
    s_items2[0] = 0;
  }
  int carry_q = 0, carry_i = 0, carry_i2 = 0;
  for (int base = 0; base < R; base += kTileThreads) {
    const int r = base + tid;
    int ql = 0, items = 0, items2 = 0;
    if (r < R) {
      const int L = clampi(a.seq_lens[r], 0, a.len_cap);
      ql = clampi(a.query_lens[r], 0, L);
      if (ql > kRowsPerUnit) {
        const int rb = (ql + kTileRows - 1) / kTileRows;
        items = rb * ((L + kPage * kRunPages - 1) / (kPage * kRunPages));
        items2 = rb * ((L + 2 * kPage * kRunPages - 1) / (2 * kPage * kRunPages));
      }
    }
    int tq, ti, ti2;
    const int eq = tile_exclusive_scan(ql, s_scan, &tq);
    const int ei = tile_exclusive_scan(items, s_scan, &ti);
    const int ei2 = tile_exclusive_scan(items2, s_scan, &ti2);
    if (r < R) {
      s_cuq[r + 1] = carry_q + eq + ql;
      s_items[r + 1] = carry_i + ei + items;
      s_items2[r + 1] = carry_i2 + ei2 + items2;
    }
    carry_q += tq;
    carry_i += ti;
    carry_i2 += ti2;
  }
  __syncthreads();
  // Runs of 16 pages when they take fewer rounds of the grid times (pages +
  // about two pages' worth of per-item start-up: the query tiles and the
  // first page, not overlapped) than runs of 8; every workgroup computes the
  // same totals, so all take the same choice.
  const int g = static_cast<int>(gridDim.x);
  const bool longer = ((s_items2[R] + g - 1) / g) * (2 * kRunPages + 2) < ((s_items[R] + g - 1) / g) * (kRunPages + 2);
  const int run_pages = longer ? 2 * kRunPages : kRunPages;
  if (longer) s_items = s_items2;
  const int total = s_items[R];

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    int lo = 0, hi = R;  // last r with s_items[r] <= item
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_items[mid] <= item) lo = mid; else hi = mid;
    }
    const int r = lo;
    const int L = clampi(a.seq_lens[r], 0, a.len_cap);
    const int ql = s_cuq[r + 1] - s_cuq[r];
    const int nb_r = (L + kPage - 1) / kPage;
    const int runs = (L + kPage * run_pages - 1) / (kPage * run_pages);
    const int local = item - s_items[r];
    const int rb = local / runs, run = local - rb * runs;
    const int j0 = run * run_pages, j1 = min(j0 + run_pages, nb_r);
    // rows of this workgroup and of this wave
    const int blk_rows = min(kTileRows, ql - rb * kTileRows);
    const int w_first = rb * kTileRows + wave * kWaveRows;      // first row (within the request)
    const int w_rows = clampi(ql - w_first, 0, kWaveRows);
    const int pos_first = L - ql + w_first;                     // its absolute position
    const int pos_blk_last = L - ql + rb * kTileRows + blk_rows - 1;
    const int jv1 = max(j0, min(j1, pos_blk_last / kPage + 1)); // pages someone in the block sees
    const int32_t* bt = a.block_table + static_cast<size_t>(r) * a.ld_bt;
    // the run's page ids, one per lane, fetched once with the item
    const int pid_lane = clampi(bt[min(j0 + (lane % run_pages), max(jv1 - 1, 0))], 0, a.num_pages - 1);
    auto page_id = [&](int j) { return __builtin_amdgcn_readlane(pid_lane, j - j0); };

    PageStage<IDX_FP8> st;
    if (j0 < jv1) st.load(a, page_id(j0), tid);
    // the wave's 64 rows as A operands (zero past the request's rows)
    bf16x8 qa[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int m = mt * 16 + (lane & 15);
      if (m < w_rows) {
        const uint16_t* qp = a.index_q + static_cast<size_t>(s_cuq[r] + w_first + m) * kDim + (lane >> 4) * 8;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) qa[mt][kc] = *reinterpret_cast<const bf16x8*>(qp + kc * 32);
      } else {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) qa[mt][kc] = bf16x8{};
      }
    }
    // the query tiles are waited for here, on every path: otherwise the
    // compiler's wait counting, merging the path with no pages, would wait
    // inside the product loop on the next page's staging loads
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) asm volatile("" ::"v"(qa[mt][kc]));
    float* srow = a.scores + static_cast<size_t>(s_cuq[r] + w_first) * a.ld_s;  // the wave's first row
    if (j0 < jv1) st.store(sh, 0, tid);
    __syncthreads();

    for (int j = j0; j < jv1; ++j) {
      const int buf = (j - j0) & 1;
      const bool next = j + 1 < jv1;
      if (next) st.load(a, page_id(j + 1), tid);  // in flight during this page's products
      if (w_rows > 0 && j * kPage <= pos_first + w_rows - 1) {
        // every row of the wave sees the whole page: no mask
        const bool whole = w_rows == kWaveRows && j * kPage + kPage - 1 <= pos_first;
        // S^T tiles: K_page rows (tokens) as the A operand, Q^T as B, so a
        // lane holds four tokens 4*(lane/16)+i of query row lane%16 and
        // keeps a running max per row tile; the four lane groups are merged
        // once per page
        float mx[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) mx[mt] = -INFINITY;
        auto column = [&](int tt, const bf16x8 (&kb)[4]) {
          f32x4 acc[4];
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < 4; ++kc)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma_16x16x32(kb[kc], qa[mt][kc], acc[mt]);
          const int t0 = j * kPage + tt * 16 + 4 * (lane >> 4);
          if (whole) {
            if constexpr (IDX_FP8 != 0) {
              const f32x4 sc = *reinterpret_cast<const f32x4*>(&sh.scale[buf][t0 - j * kPage]);
#pragma unroll
              for (int mt = 0; mt < 4; ++mt)
                mx[mt] = fmaxf(fmaxf(mx[mt], fmaxf(acc[mt][0] * sc[0], acc[mt][1] * sc[1])),
                               fmaxf(acc[mt][2] * sc[2], acc[mt][3] * sc[3]));
            } else {
#pragma unroll
              for (int mt = 0; mt < 4; ++mt)
                mx[mt] = fmaxf(fmaxf(mx[mt], fmaxf(acc[mt][0], acc[mt][1])), fmaxf(acc[mt][2], acc[mt][3]));
            }
          } else {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
              const int m = mt * 16 + (lane & 15);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float sc = IDX_FP8 ? sh.scale[buf][t0 - j * kPage + i] : 1.f;
                const bool visible = (m < w_rows) && (t0 + i <= pos_first + m);
                mx[mt] = fmaxf(mx[mt], visible ? acc[mt][i] * sc : -INFINITY);
              }
            }
          }
        };
        // two column tiles per step, the next one's LDS operands requested
        // before the current one's products (kept rolled: a full unroll
        // would hoist every operand of the page into registers)
        bf16x8 ka[4], kb2[4];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) ka[kc] = lds_operand(sh, buf, 0, kc, lane);
#pragma unroll 1
        for (int tt = 0; tt < 8; tt += 2) {
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) kb2[kc] = lds_operand(sh, buf, tt + 1, kc, lane);
          column(tt, ka);
          if (tt + 2 < 8) {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) ka[kc] = lds_operand(sh, buf, tt + 2, kc, lane);
          }
          column(tt + 1, kb2);
        }
        // merge the four lane groups (tokens), then lanes 0..15 hold the rows
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const float v = max_across_rows(mx[mt]);
          const int m = mt * 16 + lane;
          if (lane < 16 && m < w_rows) srow[static_cast<size_t>(m) * a.ld_s + j] = v;
        }
      } else {
        // no row of this wave sees the page
        for (int m = lane; m < w_rows; m += 64) srow[static_cast<size_t>(m) * a.ld_s + j] = -INFINITY;
      }
      if (next) st.store(sh, buf ^ 1, tid);
      __syncthreads();
    }
    // pages of the run past every row's position, and (last run) the tail
    const int jt1 = (run == runs - 1) ? a.ld_s : j1;
    const int width = jt1 - jv1;
    if (width > 0)
      for (int idx = lane; idx < w_rows * width; idx += 64) {
        const int m = idx / width;
        srow[static_cast<size_t>(m) * a.ld_s + jv1 + (idx - m * width)] = -INFINITY;
      }
  }
}

}  // namespace

hipError_t msa_launch_score_tile(const MsaScoreArgs& a, int num_wgs, hipStream_t s) {
  const size_t lds = sizeof(int) * 3 * static_cast<size_t>(a.num_reqs + 1);
  if (a.index_scale)
    hipLaunchKernelGGL(msa_score_tile_kernel<1>, dim3(num_wgs), dim3(kTileThreads), lds, s, a);
  else
    hipLaunchKernelGGL(msa_score_tile_kernel<0>, dim3(num_wgs), dim3(kTileThreads), lds, s, a);
  return hipGetLastError();
}

int msa_score_tile_items_bound(int64_t num_rows, int64_t blocks_bound) {
  // requests taken here have more than 64 rows each, so there are at most
  // num_rows / 65 of them, and their row blocks number at most
  // num_rows / 512 + (number of such requests)
  const int64_t row_blocks = num_rows / kTileRows + num_rows / (kRowsPerUnit + 1);
  const int64_t runs = (blocks_bound + kRunPages - 1) / kRunPages;
  const int64_t items = row_blocks * (runs > 0 ? runs : 1);
  return static_cast<int>(items > (1LL << 30) ? (1LL << 30) : items);
}

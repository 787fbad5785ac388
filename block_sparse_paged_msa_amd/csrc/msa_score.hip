// Index scores pooled per 128-token block (vLLM PR #54682 page, 功能与动机 and
// 实现拆解 item 1: the per-row decode scorer with work mapped to each request's
// real block count, index-K tiles shared by all query rows of a request).
//
// Work unit = (request r, page j, group g of up to 64 query rows of r).
// When the launch leaves requests of more than 64 rows to the tile kernel
// (msa_score_tile.hip), their units are skipped here.
// Units with g = 0 are numbered by a fixed stride, slot = r*S + j with S the
// host bound on a request's blocks, so a wave knows its page from its slot
// alone and requests the page before anything else; slots with j past the
// request's real block count are skipped. Units with g >= 1 (only requests
// with more than 64 query rows, i.e. prefill) follow, numbered by a device
// prefix over the requests. Every workgroup forms the running sums of query
// rows (and of the g >= 1 units) in LDS from seq_lens / query_lens while its
// first pages are in flight; in a launch of at most 64 rows there are no
// g >= 1 units, and the waves of every workgroup but the metadata writer sum
// the rows below their request themselves instead. In the fused decode step
// workgroup 0 also writes the batch metadata (cu_seqlens_q/k, cu_blocks,
// cu_units, row request ids and positions: vLLM PR #56170 page, 实现拆解
// items 1-3), so no separate metadata launch is needed.
//
// One wave owns one unit: it streams the 32 KiB index-K page into registers
// once, in 1 KiB fully coalesced runs thanks to the shuffled tile layout (the
// B operand of v_mfma_f32_16x16x32_bf16, token = column), and multiplies it
// with every 16-row tile of the group's index queries (the A operand), so the
// page is shared by all of the request's rows in the group. The max over the
// block's visible tokens is taken on the MFMA output, per row.
//
// An FP8 index cache (the optional FP8 index storage named on the vLLM PR
// #54682 page, 相关 PRs) holds e4m3fn codes in the same shuffled order, 16 KiB
// a page, and one fp32 scale per token: the wave streams the codes (512 B
// runs), widens them to bf16 in registers (exact), runs the same bf16 MFMA
// and multiplies each token's dot product by its scale before the max.
#include <type_traits>

#include "msa_internal.h"

using namespace msa;

namespace {

constexpr int kScoreThreads = 256;
constexpr int kWavesPerWg = kScoreThreads / 64;

struct Unit {
  int r, j, g;   // request, page inside the request, 64-row group
  int L, ql;     // request length and query rows (clamped)
  bool valid;
};

// One index-K page in registers as the B operand: column = token
// tt*16 + lane%16, K entries = dims kc*32 + 8*(lane/16) .. +7. A page is 8
// shuffled 16-token tiles [4][4][16][8], so each (tt, kc) operand is one
// contiguous run (1 KiB of bf16, or 512 B of fp8 codes).
template <int IDX_FP8>
struct IndexPage {
  using Raw = typename std::conditional<IDX_FP8 != 0, u32x2, bf16x8>::type;
  Raw k[8][4];
  float sc[8];  // fp8: scale of token tt*16 + lane%16

  __device__ __forceinline__ void load(const MsaScoreArgs& a, int page, int lane) {
    const size_t elem0 = static_cast<size_t>(page) * (kPage * kDim);
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const size_t at = elem0 + tt * (kSub * kDim) + (kc * 64 + lane) * 8;
        if constexpr (IDX_FP8 != 0)
          k[tt][kc] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(a.index_k) + at));
        else
          k[tt][kc] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(a.index_k) + at));
      }
    if constexpr (IDX_FP8 != 0) {
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) sc[tt] = a.index_scale[static_cast<size_t>(page) * kPage + tt * kSub + (lane & 15)];
    }
  }
  __device__ __forceinline__ bf16x8 op(int tt, int kc) const {
    if constexpr (IDX_FP8 != 0) {
      // widened where it is used: the empty asm keeps the compiler from
      // hoisting all 32 widened operands (128 registers) out of the row loop,
      // which leaves room for three waves per SIMD instead of two
      u32x2 r = k[tt][kc];
      asm volatile("" : "+v"(r));
      const u32x2 lo = fp8x4_to_bf16x4(r.x), hi = fp8x4_to_bf16x4(r.y);
      return __builtin_bit_cast(bf16x8, (u32x4{lo.x, lo.y, hi.x, hi.y}));
    } else {
      return k[tt][kc];
    }
  }
  __device__ __forceinline__ float scale(int tt) const {
    if constexpr (IDX_FP8 != 0) return sc[tt];
    else return 1.f;
  }
};

__device__ __forceinline__ int page_of(const MsaScoreArgs& a, const Unit& w) {
  return clampi(a.block_table[static_cast<size_t>(w.r) * a.ld_bt + w.j], 0, a.num_pages - 1);
}

// Scores of one unit once its page is in registers; q0 is the request's first row.
template <int IDX_FP8>
__device__ __forceinline__ void score_unit(const MsaScoreArgs& a, const Unit& w, int q0, const IndexPage<IDX_FP8>& kb,
                                           int lane) {
  const int g0 = w.g * kRowsPerUnit;
  const int nrows = min(kRowsPerUnit, w.ql - g0);
  const int row0 = q0 + g0;                 // first query row of the group
  const int pos0 = w.L - w.ql + g0;         // its absolute position
  const int nb_r = (w.L + kPage - 1) / kPage;
  const int t_base = w.j * kPage + (lane & 15);
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
      for (int kc = 0; kc < 4; ++kc) acc = mfma_16x16x32(qa[kc], kb.op(tt, kc), acc);
      const int t = t_base + tt * 16;
      const float sc = kb.scale(tt);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mt * 16 + 4 * (lane >> 4) + i;
        const bool visible = (m < nrows) && (t <= pos0 + m);
        mx[i] = fmaxf(mx[i], visible ? acc[i] * sc : -INFINITY);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) mx[i] = max16(mx[i]);
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mt * 16 + 4 * (lane >> 4) + i;
        if (m < nrows && row0 + m < a.num_rows)
          a.scores[static_cast<size_t>(row0 + m) * a.ld_s + w.j] = mx[i];
      }
    }
  }
  // the unit of the request's last page also writes the -inf tail of its rows
  if (w.j == nb_r - 1) {
    const int width = a.ld_s - nb_r;
    for (int idx = lane; idx < nrows * width; idx += 64) {
      const int m = idx / width;
      const int b = nb_r + (idx - m * width);
      if (row0 + m < a.num_rows) a.scores[static_cast<size_t>(row0 + m) * a.ld_s + b] = -INFINITY;
    }
  }
}

// What a first-group slot's validity and page depend on, loaded together:
// the request's raw lengths and the slot's raw block-table entry (a slot at
// or past slots_a loads nothing).
struct SlotHead {
  int r, j;
  int L, ql, bt;
};

__device__ __forceinline__ SlotHead slot_head(const MsaScoreArgs& a, int u) {
  SlotHead h = {0, 0, 0, 0, 0};
  if (u < a.num_reqs * a.blocks_per_req) {
    h.r = u / a.blocks_per_req;
    h.j = u - h.r * a.blocks_per_req;
    h.L = a.seq_lens[h.r];
    h.ql = a.query_lens[h.r];
    h.bt = a.block_table[static_cast<size_t>(h.r) * a.ld_bt + h.j];
  }
  return h;
}

// The unit of a first-group slot r*S + j.
__device__ __forceinline__ Unit head_unit(const MsaScoreArgs& a, const SlotHead& h) {
  Unit w;
  w.r = h.r;
  w.j = h.j;
  w.g = 0;
  w.L = clampi(h.L, 0, a.len_cap);
  w.ql = clampi(h.ql, 0, w.L);
  w.valid = w.ql > 0 && w.j * kPage < w.L && !(a.skip_big && w.ql > kRowsPerUnit);
  return w;
}

// Extra row groups (g >= 1): the prefix over requests numbers them; the
// request's lengths come from the prefix in LDS.
__device__ __forceinline__ Unit extra_unit(const MsaScoreArgs& a, const int* s_extra, const int* s_cuq,
                                           const int* s_ctx0, int ue) {
  int lo = 0, hi = a.num_reqs;  // last r with extra[r] <= ue
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_extra[mid] <= ue) lo = mid; else hi = mid;
  }
  Unit w;
  w.r = lo;
  w.ql = s_cuq[lo + 1] - s_cuq[lo];
  w.L = s_ctx0[lo] + w.ql;
  const int more = (w.ql + kRowsPerUnit - 1) / kRowsPerUnit - 1;  // groups 1..more
  const int local = ue - s_extra[lo];
  w.j = more > 0 ? local / more : 0;
  w.g = more > 0 ? 1 + (local - w.j * more) : 0;
  w.valid = more > 0 && ue < s_extra[a.num_reqs];
  return w;
}

template <int IDX_FP8>
__global__ __launch_bounds__(kScoreThreads) void msa_score_kernel(MsaScoreArgs a) {
  extern __shared__ int s_dyn[];  // [R+1] row prefix, [R+1] extra-group prefix, [R] context lengths
  __shared__ int s_tot[kWavesPerWg][5];
  int* s_cuq = s_dyn;
  int* s_extra = s_dyn + a.num_reqs + 1;
  int* s_ctx0 = s_dyn + 2 * (a.num_reqs + 1);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int R = a.num_reqs;
  const bool writer = a.write_meta && blockIdx.x == 0;
  const int slots_a = R * a.blocks_per_req;
  const int nwaves = gridDim.x * kWavesPerWg;
  int u = static_cast<int>(blockIdx.x) * kWavesPerWg + wave;

  // Decode-only launches (at most 64 rows in all, so no request has a row
  // group past the first) with no metadata to write need no prefix: a wave
  // sums query_lens below its request itself and never waits on a barrier.
  IndexPage<IDX_FP8> kb;
  if (!writer && a.num_rows <= kRowsPerUnit) {
    // A slot's lengths and its block-table entry are requested together (the
    // entry lies inside the table for every slot, j < S <= ld_bt, and is
    // ignored when the slot is past the request's blocks), and the next
    // slot's once the current page is requested, so a page load waits for one
    // round trip at the start and none after it. The rows below the request
    // are summed from loads issued before the page's and added after it (a
    // loop that adds as it loads would wait for them first).
    SlotHead h = slot_head(a, u);
    for (; u < slots_a; u += nwaves) {
      const Unit w = head_unit(a, h);
      const int page = clampi(h.bt, 0, a.num_pages - 1);
      if (!w.valid) {
        h = slot_head(a, u + nwaves);
        continue;
      }
      const int rl = min(lane, R - 1);
      const int ql_raw = a.query_lens[rl], l_raw = a.seq_lens[rl];
      kb.load(a, page, lane);
      h = slot_head(a, u + nwaves);
      int q0 = (lane < w.r) ? clampi(ql_raw, 0, clampi(l_raw, 0, a.len_cap)) : 0;
      for (int r = lane + 64; r < w.r; r += 64) q0 += clampi(a.query_lens[r], 0, clampi(a.seq_lens[r], 0, a.len_cap));
      q0 = __builtin_amdgcn_readlane(wave_inclusive_scan(q0), 63);
      score_unit(a, w, q0, kb, lane);
    }
    return;
  }

  // first unit of this wave: its page is requested before the prefix work
  Unit w0 = {};
  const bool first_is_a = u < slots_a;
  if (first_is_a) {
    const SlotHead h0 = slot_head(a, u);
    w0 = head_unit(a, h0);
    if (w0.valid) kb.load(a, clampi(h0.bt, 0, a.num_pages - 1), lane);
  }

  // running sums over the requests of (query rows, KV tokens, blocks, score
  // units, extra row-group units)
  if (tid == 0) {
    s_cuq[0] = 0;
    s_extra[0] = 0;
    if (writer) {
      a.cu_q[0] = 0;
      a.cu_k[0] = 0;
      a.cu_blocks[0] = 0;
      a.cu_units[0] = 0;
    }
  }
  int carry[5] = {0, 0, 0, 0, 0};
  for (int base = 0; base < R; base += kScoreThreads) {
    const int r = base + tid;
    int L = 0, ql = 0;
    if (r < R) {
      L = clampi(a.seq_lens[r], 0, a.len_cap);
      ql = clampi(a.query_lens[r], 0, L);
    }
    const int nb = (L + kPage - 1) / kPage;
    const int groups = (ql + kRowsPerUnit - 1) / kRowsPerUnit;
    int x[5] = {ql, L, nb, nb * groups, a.skip_big ? 0 : nb * max(groups - 1, 0)};
#pragma unroll
    for (int c = 0; c < 5; ++c) x[c] = wave_inclusive_scan(x[c]);
    if (lane == 63) {
#pragma unroll
      for (int c = 0; c < 5; ++c) s_tot[wave][c] = x[c];
    }
    __syncthreads();
    int pre[5], tot[5];
#pragma unroll
    for (int c = 0; c < 5; ++c) {
      pre[c] = carry[c];
      tot[c] = 0;
    }
#pragma unroll
    for (int ww = 0; ww < kWavesPerWg; ++ww)
#pragma unroll
      for (int c = 0; c < 5; ++c) {
        pre[c] += (ww < wave) ? s_tot[ww][c] : 0;
        tot[c] += s_tot[ww][c];
      }
    __syncthreads();
    if (r < R) {
      s_cuq[r + 1] = pre[0] + x[0];
      s_extra[r + 1] = pre[4] + x[4];
      s_ctx0[r] = L - ql;
      if (writer) {
        a.cu_q[r + 1] = pre[0] + x[0];
        a.cu_k[r + 1] = pre[1] + x[1];
        a.cu_blocks[r + 1] = pre[2] + x[2];
        a.cu_units[r + 1] = pre[3] + x[3];
      }
    }
#pragma unroll
    for (int c = 0; c < 5; ++c) carry[c] += tot[c];
  }
  __syncthreads();

  // per-row request id and absolute position: in a launch of more than 64
  // rows every workgroup holds the prefix, so each writes its share of the
  // rows (one workgroup alone would hold the launch open for ~8 us on a
  // step of 8198 rows); otherwise the metadata writer takes them all
  const bool spread = a.write_meta && a.num_rows > kRowsPerUnit;
  if (writer || spread) {
    const int per = spread ? (a.num_rows + static_cast<int>(gridDim.x) - 1) / static_cast<int>(gridDim.x)
                           : a.num_rows;
    const int n_lo = spread ? static_cast<int>(blockIdx.x) * per : 0;
    const int n_hi = min(n_lo + per, a.num_rows);
    for (int n = n_lo + tid; n < n_hi; n += kScoreThreads) {
      int lo = 0, hi = R;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_cuq[mid] <= n) lo = mid; else hi = mid;
      }
      // context_len + i from LDS (no dependent global load per row);
      // rows past the request's query rows stay on its last position
      const int ql = s_cuq[lo + 1] - s_cuq[lo];
      a.row_req[n] = lo;
      a.row_pos[n] = s_ctx0[lo] + min(n - s_cuq[lo], ql - 1);
    }
  }

  if (first_is_a) {
    if (w0.valid) score_unit(a, w0, s_cuq[w0.r], kb, lane);
    u += nwaves;
  }
  const int total = slots_a + s_extra[R];
  for (; u < total; u += nwaves) {
    Unit w;
    int page;
    if (u < slots_a) {  // lengths and block-table entry requested together
      const SlotHead h = slot_head(a, u);
      w = head_unit(a, h);
      page = clampi(h.bt, 0, a.num_pages - 1);
    } else {
      w = extra_unit(a, s_extra, s_cuq, s_ctx0, u - slots_a);
      page = w.valid ? page_of(a, w) : 0;
    }
    if (!w.valid) continue;
    kb.load(a, page, lane);
    score_unit(a, w, s_cuq[w.r], kb, lane);
  }
}

}  // namespace

hipError_t msa_launch_score(const MsaScoreArgs& a, int num_wgs, hipStream_t s) {
  const size_t lds = sizeof(int) * 3 * static_cast<size_t>(a.num_reqs + 1);
  if (a.index_scale)
    hipLaunchKernelGGL(msa_score_kernel<1>, dim3(num_wgs), dim3(kScoreThreads), lds, s, a);
  else
    hipLaunchKernelGGL(msa_score_kernel<0>, dim3(num_wgs), dim3(kScoreThreads), lds, s, a);
  return hipGetLastError();
}

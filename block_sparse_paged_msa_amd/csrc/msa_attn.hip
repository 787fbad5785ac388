// Sparse paged attention over a page-16 block table with an online softmax
// (vLLM PR #47287 page, 功能与动机: attention over the few logical blocks the
// indexer selected; 实现拆解 item 2: FP8 K/V with k_scale / v_scale, scalar or
// per-token-head; 实现拆解 item 3: paged attention on the page-16 view of the
// page-128 cache).
//
// Workgroup = (row, group of 16 query heads, split of split_tok tokens), four
// waves that each walk a contiguous run of 16-token sub-pages, two at a time,
// with the next two sub-pages' loads in flight while the current pair is used:
//   S^T[token][head] = K_sub (16x128) . Q^T (128x16)   v_mfma_f32_16x16x32_bf16
//   O^T[dim][head]  += V_sub^T (128x16) . P^T (16x16)  v_mfma_f32_16x16x16_bf16
// The S^T output layout (lane = head, four tokens per lane) is exactly the
// P^T operand layout of the second product, and V sub-pages are stored
// dim-major so each lane reads its four tokens of one dim as 8 contiguous
// bytes. FP8 codes are widened to bf16 in registers (exact); a per-token K
// scale multiplies the logit, a per-token V scale multiplies the probability
// fed to the PV product; scalar scales fold into the logit scale and the final
// normalisation. The four waves merge through LDS. A row split over several
// workgroups leaves one partial (max, sum, unnormalised output) per split;
// msa_merge_kernel combines them after the kernel boundary, in split order.
//
// In the fused decode step (vLLM PR #54682 page, 实现拆解 items 1-3: the
// indexer's selection feeds attention in the same step) every workgroup
// selects its row's blocks from the block scores itself (msa_select.h): the
// selection is deterministic, so all workgroups of a row agree, and no
// workgroup waits for another. The first workgroup of each row also writes the
// page-16 table, the context length and the selected block ids.
#include "msa_select.h"

using namespace msa;

namespace {

constexpr int kAttnThreads = 256;
constexpr int kPartStride = 2 * kHeadTile + kHeadTile * kDim;  // m[16], l[16], acc[16][128]
constexpr int kLdsRow = kDim + 4;                               // padded [head][dim] rows
constexpr int kMaxSplitBlocks = kMaxSplitTokens / kPage;

template <int KV_FP8, int SCALE_MODE>
struct SubPage {
  bf16x8 k[4];   // A operand of S^T: token lane%16, dims kc*32 + 8*(lane/16)..+7
  i16x4 v[8];    // A operand of O^T: dim dt*16 + lane%16, tokens 4*(lane/16)..+3
  f32x4 ks, vs;  // per-token scales of tokens 4*(lane/16)..+3
};

template <int KV_FP8, int SCALE_MODE>
__device__ __forceinline__ void load_sub(const MsaAttnArgs& a, int sub, int lane, SubPage<KV_FP8, SCALE_MODE>& s) {
  const size_t base = static_cast<size_t>(sub) * (kSub * kDim);
  // K sub-pages are shuffled tiles [4][4][16][8]: operand kc of lane l is the
  // 8 elements at (kc*64 + l)*8, so every operand load is one contiguous run.
  if constexpr (!KV_FP8) {
    const uint16_t* kp = static_cast<const uint16_t*>(a.k_cache) + base + lane * 8;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) s.k[kc] = *reinterpret_cast<const bf16x8*>(kp + kc * 512);
    const uint16_t* vp = static_cast<const uint16_t*>(a.v_cache) + base + (lane & 15) * kSub + (lane >> 4) * 4;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) s.v[dt] = *reinterpret_cast<const i16x4*>(vp + dt * 16 * kSub);
  } else {
    const uint8_t* kp = static_cast<const uint8_t*>(a.k_cache) + base + lane * 8;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(kp + kc * 512);
      const u32x2 lo = fp8x4_to_bf16x4(w.x), hi = fp8x4_to_bf16x4(w.y);
      s.k[kc] = __builtin_bit_cast(bf16x8, (u32x4{lo.x, lo.y, hi.x, hi.y}));
    }
    const uint8_t* vp = static_cast<const uint8_t*>(a.v_cache) + base + (lane & 15) * kSub + (lane >> 4) * 4;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      s.v[dt] = __builtin_bit_cast(i16x4, fp8x4_to_bf16x4(*reinterpret_cast<const uint32_t*>(vp + dt * 16 * kSub)));
  }
  if constexpr (SCALE_MODE == 2) {
    s.ks = *reinterpret_cast<const f32x4*>(a.k_scale + static_cast<size_t>(sub) * kSub + (lane >> 4) * 4);
    s.vs = *reinterpret_cast<const f32x4*>(a.v_scale + static_cast<size_t>(sub) * kSub + (lane >> 4) * 4);
  } else {
    s.ks = f32x4{1.f, 1.f, 1.f, 1.f};
    s.vs = f32x4{1.f, 1.f, 1.f, 1.f};
  }
}

// Per-wave online-softmax state: O^T accumulators, running max (log2 domain,
// equal in the four lanes of a head) and this lane's partial denominator.
struct WaveState {
  f32x4 o[8];
  float m;
  float l;
};

// One or two consecutive sub-pages: logits, one max update, PV products.
template <int KV_FP8, int SCALE_MODE>
__device__ __forceinline__ void attend_pair(WaveState& st, SubPage<KV_FP8, SCALE_MODE> (&sp)[2], int nval0, int nval1,
                                            const bf16x8 (&qb)[4], float zscale, int lane) {
  const int tok0 = 4 * (lane >> 4);
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) s0 = mfma_16x16x32(sp[0].k[kc], qb[kc], s0);
  if (nval1 > 0) {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) s1 = mfma_16x16x32(sp[1].k[kc], qb[kc], s1);
  }
  float z0[4], z1[4], mloc = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z0[i] = (tok0 + i < nval0) ? s0[i] * zscale * sp[0].ks[i] : -INFINITY;
    z1[i] = (tok0 + i < nval1) ? s1[i] * zscale * sp[1].ks[i] : -INFINITY;
    mloc = fmaxf(mloc, fmaxf(z0[i], z1[i]));
  }
  const float m_new = fmaxf(st.m, max_across_rows(mloc));  // finite: token 0 of sub-page 0 is valid
  const float alpha = fast_exp2(st.m - m_new);
  float psum = 0.f;
  i16x4 p0, p1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float e0 = fast_exp2(z0[i] - m_new);
    const float e1 = fast_exp2(z1[i] - m_new);
    psum += e0 + e1;
    p0[i] = static_cast<short>(f32_to_bf16(e0 * sp[0].vs[i]));
    p1[i] = static_cast<short>(f32_to_bf16(e1 * sp[1].vs[i]));
  }
  st.l = st.l * alpha + psum;
  st.m = m_new;
  // V slots past the context can hold anything (even NaN codes): zero them so
  // that a zero probability cannot meet a NaN in the product.
  if (nval0 < kSub) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tok0 + i >= nval0) sp[0].v[dt][i] = 0;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.o[dt] = mfma_16x16x16(sp[0].v[dt], p0, st.o[dt] * alpha);
  if (nval1 > 0) {
    if (nval1 < kSub) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tok0 + i >= nval1) sp[1].v[dt][i] = 0;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] = mfma_16x16x16(sp[1].v[dt], p1, st.o[dt]);
  }
}

struct MergeLds {
  float m[4][kHeadTile];
  float l[4][kHeadTile];
  __attribute__((aligned(16))) float o[4][kHeadTile][kLdsRow];
};

__device__ __forceinline__ u32x4 pack_bf16x8(f32x4 a, f32x4 b, float s) {
  u32x4 pk;
  pk.x = f32_to_bf16(a.x * s) | (static_cast<uint32_t>(f32_to_bf16(a.y * s)) << 16);
  pk.y = f32_to_bf16(a.z * s) | (static_cast<uint32_t>(f32_to_bf16(a.w * s)) << 16);
  pk.z = f32_to_bf16(b.x * s) | (static_cast<uint32_t>(f32_to_bf16(b.y * s)) << 16);
  pk.w = f32_to_bf16(b.z * s) | (static_cast<uint32_t>(f32_to_bf16(b.w * s)) << 16);
  return pk;
}

// Attention of (row n, head group hgi, split) over tokens
// [split*split_tok, min(ctx, (split+1)*split_tok)); get_sub(sp) gives the
// physical sub-page of the row's sp-th sub-page. Writes the output when the
// row has one split, else this split's partial.
// Q^T as the B operand of S^T: column = head lane%16, K entries = dims
// kc*32 + 8*(lane/16)..+7 (heads past the group's end read as zero).
__device__ __forceinline__ void load_q(const MsaAttnArgs& a, int n, int hgi, bf16x8 (&qb)[4]) {
  const int lane = threadIdx.x & 63;
  const int nheads = min(kHeadTile, a.num_q_heads - hgi * kHeadTile);
  if ((lane & 15) < nheads) {
    const uint16_t* qp =
        a.q + (static_cast<size_t>(n) * a.num_q_heads + hgi * kHeadTile + (lane & 15)) * kDim + (lane >> 4) * 8;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qb[kc] = *reinterpret_cast<const bf16x8*>(qp + kc * 32);
  } else {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qb[kc] = bf16x8{};
  }
}

template <int KV_FP8, int SCALE_MODE, typename GetSub>
__device__ __forceinline__ void attend_split(const MsaAttnArgs& a, MergeLds& ml, int n, int hgi, int split, int ctx,
                                             const bf16x8 (&qb)[4], GetSub get_sub) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nsplit_n = (ctx + a.split_tok - 1) / a.split_tok;
  const int nheads = min(kHeadTile, a.num_q_heads - hgi * kHeadTile);
  uint16_t* orow = a.out + (static_cast<size_t>(n) * a.num_q_heads + hgi * kHeadTile) * kDim;
  const int th = tid >> 4;         // output / partial mapping: head th, dims td .. td+7
  const int td = (tid & 15) * 8;

  float kscal = 1.f, vscal = 1.f;
  if constexpr (SCALE_MODE == 1) {
    kscal = a.k_scale[0];
    vscal = a.v_scale[0];
  }
  const float zscale = a.scale_log2 * kscal;

  const int sp_per_wave = a.split_tok / (4 * kSub);
  const int sp_begin = split * (a.split_tok / kSub) + wave * sp_per_wave;
  const int sp_end = min(sp_begin + sp_per_wave, (ctx + kSub - 1) / kSub);

  WaveState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto nval = [&](int sp) { return sp < sp_end ? min(kSub, ctx - sp * kSub) : 0; };
  SubPage<KV_FP8, SCALE_MODE> A[2], B[2];
  int sp = sp_begin;
  if (sp < sp_end) {
    load_sub(a, get_sub(sp), lane, A[0]);
    if (sp + 1 < sp_end) load_sub(a, get_sub(sp + 1), lane, A[1]);
  }
  while (sp < sp_end) {
    if (sp + 2 < sp_end) {
      load_sub(a, get_sub(sp + 2), lane, B[0]);
      if (sp + 3 < sp_end) load_sub(a, get_sub(sp + 3), lane, B[1]);
    }
    attend_pair(st, A, nval(sp), nval(sp + 1), qb, zscale, lane);
    sp += 2;
    if (sp >= sp_end) break;
    if (sp + 2 < sp_end) {
      load_sub(a, get_sub(sp + 2), lane, A[0]);
      if (sp + 3 < sp_end) load_sub(a, get_sub(sp + 3), lane, A[1]);
    }
    attend_pair(st, B, nval(sp), nval(sp + 1), qb, zscale, lane);
    sp += 2;
  }

  // ---- merge the four waves through LDS ([head][dim] rows) ----
  const float l_w = sum_across_rows(st.l);
  if (lane < kHeadTile) {
    ml.m[wave][lane] = st.m;
    ml.l[wave][lane] = l_w;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) ml.o[wave][lane & 15][dt * 16 + 4 * (lane >> 4) + i] = st.o[dt][i];
  __syncthreads();

  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, ml.m[w][th]);
  float Lsum = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float wt = (ml.m[w][th] == -INFINITY) ? 0.f : fast_exp2(ml.m[w][th] - M);
    Lsum += wt * ml.l[w][th];
    acc0 += wt * *reinterpret_cast<const f32x4*>(&ml.o[w][th][td]);
    acc1 += wt * *reinterpret_cast<const f32x4*>(&ml.o[w][th][td + 4]);
  }

  if (nsplit_n == 1) {
    const float inv = (Lsum > 0.f) ? vscal / Lsum : 0.f;
    if (th < nheads) *reinterpret_cast<u32x4*>(orow + th * kDim + td) = pack_bf16x8(acc0, acc1, inv);
    return;
  }
  // partial: a scalar V scale is folded in here (the merge is linear in acc)
  float* part = a.partials + ((static_cast<size_t>(n) * a.num_hgroups + hgi) * a.nsplit + split) * kPartStride;
  if ((tid & 15) == 0) {
    part[th] = M;
    part[kHeadTile + th] = Lsum;
  }
  *reinterpret_cast<f32x4*>(part + 2 * kHeadTile + th * kDim + td) = acc0 * vscal;
  *reinterpret_cast<f32x4*>(part + 2 * kHeadTile + th * kDim + td + 4) = acc1 * vscal;
}

__device__ __forceinline__ void write_zero_row(const MsaAttnArgs& a, int n, int hgi) {
  const int th = threadIdx.x >> 4, td = (threadIdx.x & 15) * 8;
  const int nheads = min(kHeadTile, a.num_q_heads - hgi * kHeadTile);
  uint16_t* orow = a.out + (static_cast<size_t>(n) * a.num_q_heads + hgi * kHeadTile) * kDim;
  if (th < nheads) *reinterpret_cast<u32x4*>(orow + th * kDim + td) = u32x4{0u, 0u, 0u, 0u};
}

// Table mode: the row's sub-pages and context length come from the caller.
// Q and the split's table entries are fetched together at the start.
template <int KV_FP8, int SCALE_MODE>
__global__ __launch_bounds__(kAttnThreads) void msa_attn_table_kernel(MsaAttnArgs a) {
  __shared__ MergeLds ml;
  __shared__ int s_sub[kMaxSplitTokens / kSub];
  const int split = blockIdx.x % a.nsplit;
  const int rest = blockIdx.x / a.nsplit;
  const int hgi = rest % a.num_hgroups;
  const int n = rest / a.num_hgroups;
  const int ctx = clampi(a.ctx_in[n], 0, min(a.max_ctx, kSub * a.ld_table));
  if (ctx == 0) {
    if (split == 0) write_zero_row(a, n, hgi);
    return;
  }
  if (split * a.split_tok >= ctx) return;
  bf16x8 qb[4];
  load_q(a, n, hgi, qb);
  const int sp0 = split * (a.split_tok / kSub);
  const int nsp = min(a.split_tok / kSub, (ctx + kSub - 1) / kSub - sp0);
  const int32_t* trow = a.table_in + static_cast<size_t>(n) * a.ld_table + sp0;
  for (int i = threadIdx.x; i < nsp; i += kAttnThreads) s_sub[i] = clampi(trow[i], 0, a.num_subpages - 1);
  __syncthreads();
  attend_split<KV_FP8, SCALE_MODE>(a, ml, n, hgi, split, ctx, qb, [&](int sp) { return s_sub[sp - sp0]; });
}

// Fused mode: select the row's blocks from its scores, then attend. The
// row's keys and block-table entries sit in dynamic LDS; every wave runs the
// selection itself (wave_select / wave_compact) and keeps only the pages of
// its own sub-pages, so the waves need no barrier between selection and
// attention. The merge buffers reuse the key area afterwards. KEY_REGS keys
// per lane stay in registers during the selection (64*KEY_REGS blocks).
template <int KV_FP8, int SCALE_MODE, int KEY_REGS>
__global__ __launch_bounds__(kAttnThreads) void msa_attn_select_kernel(MsaAttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t s_dyn[];  // keys[nbmax], pages[nbmax] | MergeLds
  __shared__ int s_hist[4][256];
  __shared__ int s_wpage[4][kMaxSplitBlocks];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x % a.nsplit;
  const int rest = blockIdx.x / a.nsplit;
  const int hgi = rest % a.num_hgroups;
  const int n = rest / a.num_hgroups;
  const int nbmax = min(min(a.ld_s, a.ld_bt), kMaxBlocksPerRow);
  // round 1: the whole score row (nb <= nbmax is not known yet), the row's
  // request and position, and Q; round 2: the block-table entries, held in
  // registers while the waves run the radix passes
  const float* srow = a.scores + static_cast<size_t>(n) * a.ld_s;
  uint32_t* keys = s_dyn;
  int* pages = reinterpret_cast<int*>(s_dyn + nbmax);
  for (int e = tid; e < nbmax; e += kAttnThreads) keys[e] = order_key(srow[e]);
  const int r = clampi(a.row_req[n], 0, a.num_reqs - 1);
  const int v = a.row_pos[n] + 1;
  bf16x8 qb[4];
  load_q(a, n, hgi, qb);
  const int nb = clampi((v + kPage - 1) / kPage, 0, nbmax);
  const int32_t* bt = a.block_table + static_cast<size_t>(r) * a.ld_bt;
  constexpr int kRegBlocks = 4;  // block-table entries held per thread during the selection
  int btreg[kRegBlocks];
#pragma unroll
  for (int i = 0; i < kRegBlocks; ++i) btreg[i] = (tid + i * kAttnThreads < nb) ? bt[tid + i * kAttnThreads] : 0;
  __syncthreads();  // keys visible

  WaveKeys<KEY_REGS> wk;
  wave_load_keys(keys, nb, wk);
  const WaveSelection ws = wave_select(keys, wk, nb, a.topk, s_hist[wave]);
#pragma unroll
  for (int i = 0; i < kRegBlocks; ++i)
    if (tid + i * kAttnThreads < nb) pages[tid + i * kAttnThreads] = btreg[i];
  for (int e = tid + kRegBlocks * kAttnThreads; e < nb; e += kAttnThreads) pages[e] = bt[e];
  __syncthreads();  // pages visible
  // this wave's sub-pages and the blocks they fall in
  const int sp_per_wave = a.split_tok / (4 * kSub);
  const int sp_begin = split * (a.split_tok / kSub) + wave * sp_per_wave;
  const int wblk0 = sp_begin >> 3;
  const int wnblk = max(1, sp_per_wave >> 3);
  const bool writer = split == 0 && hgi == 0 && wave == 0;
  int32_t* trow = a.table_out + static_cast<size_t>(n) * (8 * a.topk);
  int32_t* selrow = a.sel_out ? a.sel_out + static_cast<size_t>(n) * a.topk : nullptr;
  const int pmax = a.num_subpages / kSubsPerPage - 1;
  int ctx = wave_compact(keys, wk, nb, v, ws, [&](int pos, int e) {
    const int page = pages[e];
    if (pos >= wblk0 && pos < wblk0 + wnblk) s_wpage[wave][pos - wblk0] = clampi(page, 0, pmax);
    if (writer) {
#pragma unroll
      for (int i = 0; i < 8; ++i) trow[8 * pos + i] = 8 * page + i;
      if (selrow) selrow[pos] = e;
    }
  });
  if (writer) {
    for (int m = 8 * ws.kk + lane; m < 8 * a.topk; m += 64) trow[m] = 0;
    if (selrow)
      for (int m = ws.kk + lane; m < a.topk; m += 64) selrow[m] = -1;
    if (lane == 0) a.ctx_out[n] = ctx;
  }
  __syncthreads();  // keys / pages are dead; the merge buffers may reuse them
  ctx = min(ctx, a.max_ctx);
  if (ctx == 0) {
    if (split == 0) write_zero_row(a, n, hgi);
    return;
  }
  if (split * a.split_tok >= ctx) return;
  attend_split<KV_FP8, SCALE_MODE>(a, *reinterpret_cast<MergeLds*>(s_dyn), n, hgi, split, ctx, qb,
                                   [&](int sp) { return 8 * s_wpage[wave][(sp >> 3) - wblk0] + (sp & 7); });
}

// Combines the split partials of rows that needed more than one split, in
// split order (log2-domain weights 2^(m_s - max)).
__global__ __launch_bounds__(kAttnThreads) void msa_merge_kernel(MsaAttnArgs a, const int32_t* ctxp) {
  const int tid = threadIdx.x;
  const int hgi = blockIdx.x % a.num_hgroups;
  const int n = blockIdx.x / a.num_hgroups;
  const int th = tid >> 4, td = (tid & 15) * 8;
  const float* base = a.partials + (static_cast<size_t>(n) * a.num_hgroups + hgi) * a.nsplit * kPartStride;
  // the first sixteen partials are requested in the same round as ctx (every
  // slot below nsplit exists in the workspace; unused ones are ignored)
  constexpr int kBatch = 16;
  float ms[kBatch], ls[kBatch];
  f32x4 x0[kBatch], x1[kBatch];
  auto fetch = [&](int s0) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float* ps = base + static_cast<size_t>(min(s0 + j, a.nsplit - 1)) * kPartStride;
      ms[j] = ps[th];
      ls[j] = ps[kHeadTile + th];
      x0[j] = *reinterpret_cast<const f32x4*>(ps + 2 * kHeadTile + th * kDim + td);
      x1[j] = *reinterpret_cast<const f32x4*>(ps + 2 * kHeadTile + th * kDim + td + 4);
    }
  };
  fetch(0);
  const int ctx = clampi(ctxp[n], 0, min(a.max_ctx, kSub * a.ld_table));
  const int nsplit_n = (ctx + a.split_tok - 1) / a.split_tok;
  if (nsplit_n <= 1) return;
  float Mg = -INFINITY, Lg = 0.f;
  f32x4 g0 = {0.f, 0.f, 0.f, 0.f}, g1 = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit_n; s0 += kBatch) {
    if (s0 > 0) fetch(s0);
    // batch max first, so the sixteen weights are independent of each other
    float mb = -INFINITY;
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (s0 + j < nsplit_n) mb = fmaxf(mb, ms[j]);
    const float mn = fmaxf(Mg, mb);
    const float c_old = fast_exp2(Mg - mn);  // 0 on the first batch (Mg = -inf)
    float lb = 0.f;
    f32x4 b0 = {0.f, 0.f, 0.f, 0.f}, b1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float wj = (s0 + j < nsplit_n) ? fast_exp2(ms[j] - mn) : 0.f;
      lb += ls[j] * wj;
      b0 += x0[j] * wj;
      b1 += x1[j] * wj;
    }
    Lg = Lg * c_old + lb;
    g0 = g0 * c_old + b0;
    g1 = g1 * c_old + b1;
    Mg = mn;
  }
  const int nheads = min(kHeadTile, a.num_q_heads - hgi * kHeadTile);
  uint16_t* orow = a.out + (static_cast<size_t>(n) * a.num_q_heads + hgi * kHeadTile) * kDim;
  const float inv = (Lg > 0.f) ? 1.f / Lg : 0.f;
  if (th < nheads) *reinterpret_cast<u32x4*>(orow + th * kDim + td) = pack_bf16x8(g0, g1, inv);
}

template <int KV_FP8, int SCALE_MODE>
hipError_t launch(const MsaAttnArgs& a, hipStream_t s) {
  const int64_t grid = static_cast<int64_t>(a.num_rows) * a.num_hgroups * a.nsplit;
  if (a.scores) {
    const size_t nbmax = static_cast<size_t>(min(min(a.ld_s, a.ld_bt), kMaxBlocksPerRow));
    const size_t lds = max(2 * nbmax * sizeof(uint32_t), sizeof(MergeLds));
    if (nbmax <= 256)
      hipLaunchKernelGGL((msa_attn_select_kernel<KV_FP8, SCALE_MODE, 4>), dim3(static_cast<unsigned>(grid)),
                         dim3(kAttnThreads), lds, s, a);
    else
      hipLaunchKernelGGL((msa_attn_select_kernel<KV_FP8, SCALE_MODE, 16>), dim3(static_cast<unsigned>(grid)),
                         dim3(kAttnThreads), lds, s, a);
  }
  else
    hipLaunchKernelGGL((msa_attn_table_kernel<KV_FP8, SCALE_MODE>), dim3(static_cast<unsigned>(grid)),
                       dim3(kAttnThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t msa_launch_attn(const MsaAttnArgs& a, int kv_dtype, int scale_mode, hipStream_t s) {
  if (kv_dtype == 0) {
    if (scale_mode == 0) return launch<0, 0>(a, s);
    if (scale_mode == 1) return launch<0, 1>(a, s);
    return launch<0, 2>(a, s);
  }
  if (scale_mode == 1) return launch<1, 1>(a, s);
  return launch<1, 2>(a, s);
}

hipError_t msa_launch_merge(const MsaAttnArgs& a, hipStream_t s) {
  if (a.nsplit <= 1) return hipSuccess;
  const int64_t grid = static_cast<int64_t>(a.num_rows) * a.num_hgroups;
  hipLaunchKernelGGL(msa_merge_kernel, dim3(static_cast<unsigned>(grid)), dim3(kAttnThreads), 0, s, a,
                     a.scores ? static_cast<const int32_t*>(a.ctx_out) : a.ctx_in);
  return hipGetLastError();
}

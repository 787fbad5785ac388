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
// workgroups leaves one partial per split, in the block-major path's slot
// format: max and sum in fp32 and the unnormalised output in fp16, scaled by
// a power of two that puts each head's largest magnitude in [1/2, 1) (the
// exponent folded into the max and the sum); msa_merge_kernel combines them
// after the kernel boundary, in split order.
//
// Optional extras (vLLM PR #54404 page, 实现拆解 items 1-2): the natural-log
// log-sum-exp of each (row, head)'s scaled logits, ln 2 * (m + log2 l) in the
// log2-domain state, and one sink logit per query head that adds
// 2^(sink*log2(e) - m) to the final denominator (the LSE excludes it).
//
// In the fused decode step (vLLM PR #54682 page, 实现拆解 items 1-3: the
// indexer's selection feeds attention in the same step) every workgroup
// selects its row's blocks from the block scores itself (msa_select.h): the
// selection is deterministic, so all workgroups of a row agree, and no
// workgroup waits for another. The first workgroup of each row also writes the
// page-16 table, the context length and the selected block ids.
#include <type_traits>

#include "msa_select.h"

using namespace msa;

namespace {

constexpr int kAttnThreads = 256;
constexpr int kHalfPartStride = 2 * kHeadTile + kHeadTile * kDim / 2;  // m[16], l[16], fp16 acc[16][128]
constexpr int kLdsRow = kDim + 4;                               // padded [head][dim] rows
constexpr int kMaxSplitBlocks = kMaxSplitTokens / kPage;

// 4x4 transpose of (register, 16-lane row) with the row swaps of gfx950:
// afterwards register r of lane (row g, column c) holds what register g of
// lane (row r, column c) held.
__device__ __forceinline__ void transpose_rows4(uint32_t& r0, uint32_t& r1, uint32_t& r2, uint32_t& r3) {
  auto s32 = [](uint32_t& a, uint32_t& b) {  // rows 2, 3 of a <-> rows 0, 1 of b
    const auto p = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = p[0];
    b = p[1];
  };
  auto s16 = [](uint32_t& a, uint32_t& b) {  // rows 1, 3 of a <-> rows 0, 2 of b
    const auto p = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = p[0];
    b = p[1];
  };
  s32(r0, r2);
  s32(r1, r3);
  s16(r0, r1);
  s16(r2, r3);
}

// One 16-token sub-page of K and V in registers, as loaded: bf16 operands, or
// the raw e4m3fn codes (half the registers), widened to bf16 at use.
// fp8 V arrives as two 16-byte runs per lane (lane l: all 16 tokens of dim l,
// then of dim 64 + l), a quarter of the load instructions of one operand
// per load; prep_v() turns them into the operands with a transpose across
// the four 16-lane rows once they are needed.
template <int KV_FP8, int SCALE_MODE>
struct SubPage {
  using KRaw = typename std::conditional<KV_FP8 != 0, u32x2, bf16x8>::type;
  using VRaw = typename std::conditional<KV_FP8 != 0, uint32_t, i16x4>::type;
  KRaw k[4];     // A operand of S^T: token lane%16, dims kc*32 + 8*(lane/16)..+7
  VRaw v[8];     // A operand of O^T: dim dt*16 + lane%16, tokens 4*(lane/16)..+3
  u32x4 vw[2];   // fp8: V as loaded (dims lane and 64 + lane, 16 tokens each)
  f32x4 ks, vs;  // per-token scales of tokens 4*(lane/16)..+3

  __device__ __forceinline__ void prep_v() {
    if constexpr (KV_FP8 != 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t r0 = vw[h].x, r1 = vw[h].y, r2 = vw[h].z, r3 = vw[h].w;
        transpose_rows4(r0, r1, r2, r3);
        v[4 * h] = r0;
        v[4 * h + 1] = r1;
        v[4 * h + 2] = r2;
        v[4 * h + 3] = r3;
      }
    }
  }

  __device__ __forceinline__ bf16x8 k_op(int kc) const {
    if constexpr (KV_FP8 != 0) {
      const u32x2 lo = fp8x4_to_bf16x4(k[kc].x), hi = fp8x4_to_bf16x4(k[kc].y);
      return __builtin_bit_cast(bf16x8, (u32x4{lo.x, lo.y, hi.x, hi.y}));
    } else {
      return k[kc];
    }
  }
  __device__ __forceinline__ i16x4 v_op(int dt) const {
    if constexpr (KV_FP8 != 0)
      return __builtin_bit_cast(i16x4, fp8x4_to_bf16x4(v[dt]));
    else
      return v[dt];
  }
};

template <int KV_FP8, int SCALE_MODE>
__device__ __forceinline__ void load_sub(const MsaAttnArgs& a, int sub, int lane, SubPage<KV_FP8, SCALE_MODE>& s) {
  using SP = SubPage<KV_FP8, SCALE_MODE>;
  using KRaw = typename SP::KRaw;
  using VRaw = typename SP::VRaw;
  constexpr int elt = KV_FP8 ? 1 : 2;  // bytes per element
  const size_t base = static_cast<size_t>(sub) * (kSub * kDim) * elt;
  // K sub-pages are shuffled tiles [4][4][16][8]: operand kc of lane l is the
  // 8 elements at (kc*64 + l)*8, so every operand load is one contiguous run.
  const char* kp = static_cast<const char*>(a.k_cache) + base + lane * 8 * elt;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) s.k[kc] = __builtin_nontemporal_load(reinterpret_cast<const KRaw*>(kp + kc * 512 * elt));
  if constexpr (KV_FP8 != 0) {
    // dim-major fp8 sub-page: dim d's 16 tokens are the 16 bytes at 16*d
    const char* vp = static_cast<const char*>(a.v_cache) + base + lane * 16;
    s.vw[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp));
    s.vw[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + 64 * kSub));
  } else {
    const char* vp = static_cast<const char*>(a.v_cache) + base + ((lane & 15) * kSub + (lane >> 4) * 4) * elt;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      s.v[dt] = __builtin_nontemporal_load(reinterpret_cast<const VRaw*>(vp + dt * 16 * kSub * elt));
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
  for (int kc = 0; kc < 4; ++kc) s0 = mfma_16x16x32(sp[0].k_op(kc), qb[kc], s0);
  if (nval1 > 0) {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) s1 = mfma_16x16x32(sp[1].k_op(kc), qb[kc], s1);
  }
  float z0[4], z1[4], mloc = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z0[i] = (tok0 + i < nval0) ? s0[i] * zscale * sp[0].ks[i] : -INFINITY;
    z1[i] = (tok0 + i < nval1) ? s1[i] * zscale * sp[1].ks[i] : -INFINITY;
    mloc = fmaxf(mloc, fmaxf(z0[i], z1[i]));
  }
  const float m_new = fmaxf(st.m, max_across_rows(mloc));  // finite: token 0 of sub-page 0 is valid
  sp[0].prep_v();
  if (nval1 > 0) sp[1].prep_v();
  const float alpha = fast_exp2(st.m - m_new);
  float psum = 0.f, e0[4], e1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e0[i] = fast_exp2(z0[i] - m_new);
    e1[i] = fast_exp2(z1[i] - m_new);
    psum += e0[i] + e1[i];
  }
  if constexpr (SCALE_MODE == 2) {
    // per-token V scales; a hidden token's scale can be anything (even NaN),
    // so its probability is set to zero rather than scaled
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e0[i] = (tok0 + i < nval0) ? e0[i] * sp[0].vs[i] : 0.f;
      e1[i] = (tok0 + i < nval1) ? e1[i] * sp[1].vs[i] : 0.f;
    }
  }
  const i16x4 p0 = __builtin_bit_cast(i16x4, (u32x2{pk_bf16(e0[0], e0[1]), pk_bf16(e0[2], e0[3])}));
  const i16x4 p1 = __builtin_bit_cast(i16x4, (u32x2{pk_bf16(e1[0], e1[1]), pk_bf16(e1[2], e1[3])}));
  st.l = st.l * alpha + psum;
  st.m = m_new;
  // V slots past the context can hold anything (even NaN codes): zero them so
  // that a zero probability cannot meet a NaN in the product.
  auto v_masked = [&](const SubPage<KV_FP8, SCALE_MODE>& x, int dt, int nval) {
    i16x4 op = x.v_op(dt);
    if (nval < kSub) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tok0 + i >= nval) op[i] = 0;
    }
    return op;
  };
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.o[dt] = mfma_16x16x16(v_masked(sp[0], dt, nval0), p0, st.o[dt] * alpha);
  if (nval1 > 0) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] = mfma_16x16x16(v_masked(sp[1], dt, nval1), p1, st.o[dt]);
  }
}

struct MergeLds {
  float m[4][kHeadTile];
  float l[4][kHeadTile];
  __attribute__((aligned(16))) float o[4][kHeadTile][kLdsRow];
};

__device__ __forceinline__ u32x4 pack_bf16x8(f32x4 a, f32x4 b, float s) {
  return u32x4{pk_bf16(a.x * s, a.y * s), pk_bf16(a.z * s, a.w * s), pk_bf16(b.x * s, b.y * s),
               pk_bf16(b.z * s, b.w * s)};
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

// Same loads in every lane: lanes past the group's heads read the group's last
// head instead of zeros (their columns are never read back), so the loads are
// issued with no branch around them.
__device__ __forceinline__ void load_q_any(const MsaAttnArgs& a, int n, int hgi, bf16x8 (&qb)[4]) {
  const int lane = threadIdx.x & 63;
  const int h = min(lane & 15, a.num_q_heads - hgi * kHeadTile - 1);
  const uint16_t* qp = a.q + (static_cast<size_t>(n) * a.num_q_heads + hgi * kHeadTile + h) * kDim + (lane >> 4) * 8;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) qb[kc] = *reinterpret_cast<const bf16x8*>(qp + kc * 32);
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
  // the sink is fetched now so that its load is long done at the end
  const float sink2 = (a.sinks && th < nheads) ? a.sinks[hgi * kHeadTile + th] * kLog2e : -INFINITY;

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
    const float den = Lsum + fast_exp2(sink2 - M);  // M is finite: the split holds a token
    const float inv = (Lsum > 0.f) ? vscal / den : 0.f;
    if (th < nheads) *reinterpret_cast<u32x4*>(orow + th * kDim + td) = pack_bf16x8(acc0, acc1, inv);
    if (a.lse_out && (tid & 15) == 0 && th < nheads)
      a.lse_out[static_cast<size_t>(n) * a.num_q_heads + hgi * kHeadTile + th] = (M + log2f(Lsum)) * kLn2;
    return;
  }
  // partial: a scalar V scale is folded in here (the merge is linear in
  // acc), with the head's exponent ex from its largest |acc| (the 16 threads
  // of a head are one 16-lane row); it is read once, by the merge, so it is
  // stored non-temporal
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fmaxf(fabsf(acc0[i]), fabsf(acc1[i])));
  mx = max16(mx) * fabsf(vscal);
  const int ex = (mx > 0.f) ? clampi(__builtin_amdgcn_frexp_expf(mx), -kHalfExpRange, kHalfExpRange) : 0;
  const float f = ldexpf(vscal, -ex);
  float* part = a.partials + ((static_cast<size_t>(n) * a.num_hgroups + hgi) * a.nsplit + split) * kHalfPartStride;
  if ((tid & 15) == 0) {
    part[th] = M + static_cast<float>(ex);
    part[kHeadTile + th] = ldexpf(Lsum, -ex);
  }
  uint16_t* acc = reinterpret_cast<uint16_t*>(part + 2 * kHeadTile) + th * kDim + td;
  __builtin_nontemporal_store(u32x4{pk_f16(acc0.x * f, acc0.y * f), pk_f16(acc0.z * f, acc0.w * f),
                                    pk_f16(acc1.x * f, acc1.y * f), pk_f16(acc1.z * f, acc1.w * f)},
                              reinterpret_cast<u32x4*>(acc));
}

__device__ __forceinline__ void write_zero_row(const MsaAttnArgs& a, int n, int hgi) {
  const int th = threadIdx.x >> 4, td = (threadIdx.x & 15) * 8;
  const int nheads = min(kHeadTile, a.num_q_heads - hgi * kHeadTile);
  uint16_t* orow = a.out + (static_cast<size_t>(n) * a.num_q_heads + hgi * kHeadTile) * kDim;
  if (th < nheads) *reinterpret_cast<u32x4*>(orow + th * kDim + td) = u32x4{0u, 0u, 0u, 0u};
  if (a.lse_out && (threadIdx.x & 15) == 0 && th < nheads)
    a.lse_out[static_cast<size_t>(n) * a.num_q_heads + hgi * kHeadTile + th] = -INFINITY;
}

// Table mode: the row's sub-pages and context length come from the caller.
// Q and the split's table entries are fetched together at the start.
template <int KV_FP8, int SCALE_MODE>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2))) void msa_attn_table_kernel(MsaAttnArgs a) {
  __shared__ MergeLds ml;
  __shared__ int s_sub[kMaxSplitTokens / kSub];
  const int split = blockIdx.x % a.nsplit;
  const int rest = blockIdx.x / a.nsplit;
  const int hgi = rest % a.num_hgroups;
  const int n = rest / a.num_hgroups;
  const int ctx = clampi(a.ctx_in[n], 0, a.max_ctx);  // the host checked max_ctx <= 16 * ld_table
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

// Fused mode, after the selection: attend over this split and write the
// selection's outputs. s_wpage / s_wsel hold the raw page and block id of the
// ranks [wblk0, wblk0 + wnblk) this wave's sub-pages fall in.
template <int KV_FP8, int SCALE_MODE>
__device__ __forceinline__ void attend_selected(const MsaAttnArgs& a, MergeLds& ml, const int* s_wpage,
                                                const int* s_wsel, int n, int hgi, int split, int sp_begin,
                                                int wblk0, int wnblk, int kk, int ctx_row, const bf16x8 (&qb)[4]) {
  const int lane = threadIdx.x & 63;
  const int pmax = a.num_subpages / kSubsPerPage - 1;
  const int ctx = min(ctx_row, a.max_ctx);
  if (ctx > 0 && split * a.split_tok < ctx)
    attend_split<KV_FP8, SCALE_MODE>(a, ml, n, hgi, split, ctx, qb, [&](int sp) {
      return 8 * clampi(s_wpage[(sp >> 3) - wblk0], 0, pmax) + (sp & 7);
    });
  else if (ctx == 0 && split == 0)
    write_zero_row(a, n, hgi);

  // The selection's outputs, written once the attention's loads are out so
  // that no wait for these stores holds them back. Rank q is written by the
  // wave whose sub-pages start its block, in head group 0 (every rank lies in
  // a split that attends, since 128*q < ctx).
  if (hgi == 0 && (sp_begin & 7) == 0) {
    int32_t* trow = a.table_out + static_cast<size_t>(n) * (8 * a.topk);
    const int nq = min(wblk0 + wnblk, kk) - wblk0;
    for (int idx = lane; idx < 8 * nq; idx += 64) trow[8 * wblk0 + idx] = 8 * s_wpage[idx >> 3] + (idx & 7);
    if (a.sel_out)
      for (int m = lane; m < nq; m += 64) a.sel_out[static_cast<size_t>(n) * a.topk + wblk0 + m] = s_wsel[m];
  }
  if (split == 0 && hgi == 0 && (threadIdx.x >> 6) == 0) {  // context length and the zero tail past K'
    int32_t* trow = a.table_out + static_cast<size_t>(n) * (8 * a.topk);
    for (int m = 8 * kk + lane; m < 8 * a.topk; m += 64) trow[m] = 0;
    if (a.sel_out)
      for (int m = kk + lane; m < a.topk; m += 64) a.sel_out[static_cast<size_t>(n) * a.topk + m] = -1;
    if (lane == 0) a.ctx_out[n] = ctx_row;
  }
}

// Fused mode for rows of at most 256*KC blocks: the four waves select
// together (coop_select / coop_locate: shared radix histogram, one barrier
// per pass), then attend.
template <int KV_FP8, int SCALE_MODE, int KC>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2))) void msa_attn_coop_kernel(MsaAttnArgs a) {
  __shared__ MergeLds ml;
  __shared__ __attribute__((aligned(16))) CoopLds cl;
  __shared__ int s_wpage[4][kMaxSplitBlocks];  // raw page of each of the wave's ranks
  __shared__ int s_wsel[4][kMaxSplitBlocks];   // and its block id
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x % a.nsplit;
  const int rest = blockIdx.x / a.nsplit;
  const int hgi = rest % a.num_hgroups;
  const int n = rest / a.num_hgroups;
  const int nbmax = min(min(a.ld_s, a.ld_bt), 256 * KC);
  // first batch of loads: the row's keys, its request and position, and Q
  // (indices clamped so that every load issues unconditionally); second: the
  // block-table entries, which arrive during the radix passes
  const float* srow = a.scores + static_cast<size_t>(n) * a.ld_s;
  float kraw[KC];
#pragma unroll
  for (int i = 0; i < KC; ++i) kraw[i] = srow[min(tid + 256 * i, max(nbmax, 1) - 1)];
  const int r = clampi(a.row_req[n], 0, a.num_reqs - 1);
  const int v = a.row_pos[n] + 1;
  bf16x8 qb[4];
  load_q(a, n, hgi, qb);
  coop_clear(cl);
  const int nb = clampi((v + kPage - 1) / kPage, 0, nbmax);
  const int32_t* bt = a.block_table + static_cast<size_t>(r) * a.ld_bt;
  int pg[KC];
#pragma unroll
  for (int i = 0; i < KC; ++i) pg[i] = bt[min(tid + 256 * i, max(nb, 1) - 1)];
  uint32_t k[KC];
#pragma unroll
  for (int i = 0; i < KC; ++i) k[i] = order_key(kraw[i]);
  const WaveSelection ws = coop_select<KC>(k, nb, a.topk, cl);
  // this wave's sub-pages and the blocks (ranks) they fall in
  const int sp_per_wave = a.split_tok / (4 * kSub);
  const int sp_begin = split * (a.split_tok / kSub) + wave * sp_per_wave;
  const int wblk0 = sp_begin >> 3;
  const int wnblk = max(1, sp_per_wave >> 3);
  const int ctx = coop_locate<KC>(k, pg, nb, v, ws, wblk0, wblk0 + wnblk, cl, [&](int q, int e, int page) {
    if (lane == 0) {
      s_wpage[wave][q - wblk0] = page;
      s_wsel[wave][q - wblk0] = e;
    }
  });
  wave_lds_order();  // this wave's pages
  attend_selected<KV_FP8, SCALE_MODE>(a, ml, s_wpage[wave], s_wsel[wave], n, hgi, split, sp_begin, wblk0, wnblk,
                                      ws.kk, ctx, qb);
}

// Fused mode for longer rows: every wave loads the row's keys and
// block-table entries into registers and runs the selection itself
// (wave_select / wave_locate), keeping only the pages of its own sub-pages,
// so nothing before the attention's own merge needs a workgroup barrier.
// KEY_REGS keys per lane sit in registers (64*KEY_REGS blocks); keys and
// pages past them are read from global memory.
template <int KV_FP8, int SCALE_MODE, int KEY_REGS>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2))) void msa_attn_select_kernel(MsaAttnArgs a) {
  __shared__ MergeLds ml;
  __shared__ __attribute__((aligned(16))) int s_hist[4][kWaveRadixPasses][256];
  __shared__ int s_wpage[4][kMaxSplitBlocks];  // raw page of each of the wave's ranks
  __shared__ int s_wsel[4][kMaxSplitBlocks];   // and its block id
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x % a.nsplit;
  const int rest = blockIdx.x / a.nsplit;
  const int hgi = rest % a.num_hgroups;
  const int n = rest / a.num_hgroups;
  const int nbmax = min(min(a.ld_s, a.ld_bt), kMaxBlocksPerRow);
  const float* srow = a.scores + static_cast<size_t>(n) * a.ld_s;
  WaveKeys<KEY_REGS> wk;
  float kraw[KEY_REGS];
#pragma unroll
  for (int i = 0; i < KEY_REGS; ++i) kraw[i] = srow[min(lane + 64 * i, max(nbmax, 1) - 1)];
  const int r = clampi(a.row_req[n], 0, a.num_reqs - 1);
  const int v = a.row_pos[n] + 1;
  bf16x8 qb[4];
  load_q(a, n, hgi, qb);
  wave_clear_hist(s_hist[wave]);
  const int nb = clampi((v + kPage - 1) / kPage, 0, nbmax);
  const int32_t* bt = a.block_table + static_cast<size_t>(r) * a.ld_bt;
  int pg[KEY_REGS];
#pragma unroll
  for (int i = 0; i < KEY_REGS; ++i) pg[i] = bt[min(lane + 64 * i, max(nb, 1) - 1)];
#pragma unroll
  for (int i = 0; i < KEY_REGS; ++i) wk.k[i] = order_key(kraw[i]);
  auto tail_key = [&](int e) { return order_key(srow[e]); };
  auto tail_page = [&](int e) { return bt[e]; };
  wave_lds_order();  // histograms cleared
  const WaveSelection ws = wave_select(wk, nb, a.topk, s_hist[wave], tail_key);
  const int sp_per_wave = a.split_tok / (4 * kSub);
  const int sp_begin = split * (a.split_tok / kSub) + wave * sp_per_wave;
  const int wblk0 = sp_begin >> 3;
  const int wnblk = max(1, sp_per_wave >> 3);
  const int ctx = wave_locate(wk, pg, nb, v, ws, wblk0, wblk0 + wnblk, tail_key, tail_page, [&](int q, int e, int page) {
    if (lane == 0) {
      s_wpage[wave][q - wblk0] = page;
      s_wsel[wave][q - wblk0] = e;
    }
  });
  wave_lds_order();  // this wave's pages
  attend_selected<KV_FP8, SCALE_MODE>(a, ml, s_wpage[wave], s_wsel[wave], n, hgi, split, sp_begin, wblk0, wnblk,
                                      ws.kk, ctx, qb);
}

// Combines the partials of rows split over several workgroups (ALL_ROWS
// false: rows of one split were written by the attention kernel) or every
// row's block partials (ALL_ROWS true: a row with no slot gets zeros). One
// wave per (row, query head): lane group g = lane/16 takes splits g, g+4,
// g+8, ... and eight dims (lane%16)*8.. of each, so one round of loads
// fetches thirty-two splits of 256 B. The four groups are then combined
// through row and half swaps. All weights are log2-domain 2^(m_s - max).
constexpr int kMergeThreads = 64;

struct MergeState {
  float m, l;
  f32x4 o0, o1;
};

// Both lanes of a swapped pair receive the same combination: the two
// operands are ordered (even row or half first) before they are added.
template <bool HALVES>
__device__ __forceinline__ MergeState merge_partner(const MergeState& x) {
  auto swap = [](float v) {
    const uint32_t u = __float_as_uint(v);
    auto p = HALVES ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                    : __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return float2{__uint_as_float(p[0]), __uint_as_float(p[1])};
  };
  const float2 m = swap(x.m), l = swap(x.l);
  const float mn = fmaxf(m.x, m.y);
  const float ca = (m.x == -INFINITY) ? 0.f : fast_exp2(m.x - mn);
  const float cb = (m.y == -INFINITY) ? 0.f : fast_exp2(m.y - mn);
  MergeState r;
  r.m = mn;
  r.l = l.x * ca + l.y * cb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float2 p = swap(x.o0[i]), q = swap(x.o1[i]);
    r.o0[i] = p.x * ca + p.y * cb;
    r.o1[i] = q.x * ca + q.y * cb;
  }
  return r;
}

template <bool ALL_ROWS>
__global__ __launch_bounds__(kMergeThreads) void msa_merge_kernel(MsaAttnArgs a, const int32_t* ctxp) {
  constexpr int kStride = kHalfPartStride;
  const int lane = threadIdx.x;
  // workgroups go to the 8 XCDs in turn: the heads of row n are numbered so
  // that they all land on XCD n % 8 and share its L2 copy of each slot's
  // m / l line
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int head = local % a.num_q_heads;
  const int n = (local / a.num_q_heads) * 8 + xcd;
  if (n >= a.num_rows) return;
  const int hgi = head / kHeadTile, th = head % kHeadTile;
  const int sg = lane >> 4, td = (lane & 15) * 8;
  const float* base = a.partials + (static_cast<size_t>(n) * a.num_hgroups + hgi) * a.nsplit * kStride;
  // the first thirty-two partials are requested in the same round as ctx
  // (every slot below nsplit exists in the workspace; unused ones are ignored).
  // Accumulators are read once: non-temporal loads (the max / sum line of a
  // slot is shared by the row's heads and stays cached)
  constexpr int kPer = 8;  // splits per lane per round
  float ms[kPer], ls[kPer];
  f32x4 x0[kPer], x1[kPer];
  auto fetch = [&](int s0) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const float* ps = base + static_cast<size_t>(min(s0 + sg + 4 * j, a.nsplit - 1)) * kStride;
      ms[j] = ps[th];
      ls[j] = ps[kHeadTile + th];
      const u32x4 h = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(ps + 2 * kHeadTile) + th * kDim + td));
      x0[j] = f32x4{f16_lo(h.x), f16_hi(h.x), f16_lo(h.y), f16_hi(h.y)};
      x1[j] = f32x4{f16_lo(h.z), f16_hi(h.z), f16_lo(h.w), f16_hi(h.w)};
    }
  };
  fetch(0);
  const float sink2 = a.sinks ? a.sinks[head] * kLog2e : -INFINITY;
  const int ctx = clampi(ctxp[n], 0, a.max_ctx);  // the host checked max_ctx <= 16 * ld_table
  const int nsplit_n = (ctx + a.split_tok - 1) / a.split_tok;
  if (!ALL_ROWS && nsplit_n <= 1) return;
  MergeState st = {-INFINITY, 0.f, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int s0 = 0; s0 < nsplit_n; s0 += 4 * kPer) {
    if (s0 > 0) fetch(s0);
    float mb = -INFINITY;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (s0 + sg + 4 * j < nsplit_n) mb = fmaxf(mb, ms[j]);
    if (mb == -INFINITY) continue;  // no split of this lane group in the round
    const float mn = fmaxf(st.m, mb);
    const float c_old = fast_exp2(st.m - mn);  // 0 while st.m = -inf
    float lb = 0.f;
    f32x4 b0 = {0.f, 0.f, 0.f, 0.f}, b1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const float wj = (s0 + sg + 4 * j < nsplit_n) ? fast_exp2(ms[j] - mn) : 0.f;
      lb += ls[j] * wj;
      b0 += x0[j] * wj;
      b1 += x1[j] * wj;
    }
    st.l = st.l * c_old + lb;
    st.o0 = st.o0 * c_old + b0;
    st.o1 = st.o1 * c_old + b1;
    st.m = mn;
  }
  st = merge_partner<false>(st);
  st = merge_partner<true>(st);
  if (sg == 0) {
    uint16_t* orow = a.out + (static_cast<size_t>(n) * a.num_q_heads + head) * kDim;
    const float den = st.l + fast_exp2(sink2 - st.m);
    const float inv = (st.l > 0.f) ? 1.f / den : 0.f;
    *reinterpret_cast<u32x4*>(orow + td) = pack_bf16x8(st.o0, st.o1, inv);
    if (a.lse_out && lane == 0)
      a.lse_out[static_cast<size_t>(n) * a.num_q_heads + head] = (st.m + log2f(st.l)) * kLn2;
  }
}

// Block-major attention for prefill-sized fused steps. A work item is
// (request r, block b of r): the workgroup finds the rows of r that selected
// b from the selection words the top-k step wrote (one 8-byte word per row
// gives both the bit and the block's rank in the row's selection), compacts
// them in row order into an LDS list, copies the block's K and V (one
// contiguous run each: its 8 sub-pages are consecutive) into LDS once if the
// list is not empty, and every wave takes one (row, head group) of the list
// at a time: all 128 tokens' logits from LDS, the block's softmax
// statistics, and the PV products. The block's partial (max, sum,
// unnormalised output) goes to the row's slot for the block's rank, and
// msa_merge_kernel combines the slots in rank order (one slot too), as it
// does for token splits, and applies sinks and the LSE output.
//
// Items differ in size (a block that many rows choose is a long list), so
// when msa_block_count_kernel has counted each item's rows the launch is
// balanced by cost, not items: an item costs kItemCost plus one per entry,
// items are laid end to end (entries in row order after the fixed part),
// and workgroup g takes the cost range [C*g/G, C*(g+1)/G) of the C in all,
// i.e. the entries of the items that fall in it; an item cut between two
// workgroups is staged by both (vLLM PR #54682 page, 实现拆解 item 1: work
// mapped to the real amount per request, here per block). Without counts,
// items go to workgroups by grid stride. Each entry writes its own slot, so
// the split changes no result.
constexpr int kBlockThreads = 256;
constexpr int kRowChunk = 1024;                           // rows of a request examined per pass
constexpr int kListRankShift = 18;                        // entry = row within the request | rank << 18
constexpr uint32_t kListRowMask = (1u << kListRankShift) - 1u;
constexpr int kListRankMax = (1 << (31 - kListRankShift)) - 1;

// The block in LDS is always bf16 (fp8 codes are widened once, when staged).
struct BlockLds {
  static constexpr int kPlane = kPage * kDim * 2;                   // bytes of one bf16 plane of a block
  __attribute__((aligned(16))) uint8_t k[kPlane];                   // 8 shuffled K tiles
  __attribute__((aligned(16))) uint8_t v[kPlane];                   // V sub-pages, dim-major, pairs interleaved
  float ks[kPage], vs[kPage];
  uint32_t vmax[4];                                                 // per wave: largest |V| bits (bf16, no scales)
  int ent[kRowChunk];                                               // (row, rank) entries of a pass
  int scan[4];                                                      // block scan scratch
  int rng[4];                                                       // balanced range: first and last item, their cost offsets
  int pcnt[kRowChunk / kBlockThreads][4];                           // hits per (row segment, wave) of a pass
};
// Cost of an item in the balanced schedule, in units of one entry: its
// entries plus a fixed cost for finding its rows (a pass per 1024 rows of
// the request) and staging its block. Measured on a step of 8198 rows
// (two 4096-row prefills among decode rows): 4 -> 1170 us, 16 -> 738,
// 32 -> 708, 48 -> 709, 64 -> 720, 96 -> 790.
constexpr int kItemCost = 32;

__device__ __forceinline__ bf16x8 lds_k_op(const BlockLds& sh, int i, int kc, int lane) {
  const int e = i * (kSub * kDim) + (kc * 64 + lane) * 8;  // element offset of the operand
  return *reinterpret_cast<const bf16x8*>(sh.k + 2 * e);
}

// V sub-pages sit in LDS dim-major, 32 B a dim (16 tokens), with the four
// 8-byte token groups of dim d stored at position g ^ ((d >> 2) & 3): the 16
// lanes that read one token group of 16 consecutive dims then hit 16
// different bank pairs instead of 4. The rows are ordered [sub-page pair]
// [16-dim tile][sub-page of the pair][16 dims], so the two halves of a PV
// operand (the same dims in sub-pages 2p and 2p+1) are 512 B apart and the
// closest pair of reads: the compiler merges exactly those two into one
// read2st64 whose destination is the operand, with no register moves.
__device__ __forceinline__ int v_swz(int d) { return (d >> 2) & 3; }

// Row (32 B) of dim d of sub-page i.
__device__ __forceinline__ int v_row(int i, int d) {
  return (i >> 1) * (2 * kDim) + (d >> 4) * 32 + (i & 1) * 16 + (d & 15);
}

__device__ __forceinline__ i16x4 lds_v_op(const BlockLds& sh, int i, int dt, int lane) {
  const int d = dt * 16 + (lane & 15);
  const int e = v_row(i, d) * kSub + 4 * ((lane >> 4) ^ v_swz(d));
  return *reinterpret_cast<const i16x4*>(sh.v + 2 * e);
}

template <int KV_FP8, int SCALE_MODE>
__global__ __launch_bounds__(kBlockThreads, 2) void msa_attn_block_kernel(MsaAttnArgs a, MsaBlockArgs bk) {
  __shared__ BlockLds sh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tok0 = 4 * (lane >> 4);
  float kscal = 1.f, vscal = 1.f;
  if constexpr (SCALE_MODE == 1) {
    kscal = a.k_scale[0];
    vscal = a.v_scale[0];
  }
  const float zscale = a.scale_log2 * kscal;
  const int pmax = a.num_subpages / kSubsPerPage - 1;
  const int items = bk.num_reqs * bk.nbmax;

  // this workgroup's items: a grid stride, or with counts the items its cost
  // range [A, B) meets (the first and the last of them only partly)
  int it_begin = blockIdx.x, it_stop = items, it_step = gridDim.x;
  int64_t cost_a = 0, cost_b = 0, p_first = 0, p_last = 0;  // range; cost offsets of its first / last item
  auto item_cost = [](int c) { return c > 0 ? c + kItemCost : 0; };
  if (bk.counts) {
    int64_t t = 0;
    for (int i = tid; i < items; i += kBlockThreads) t += item_cost(bk.counts[i]);
    // the total, summed as two 16-bit halves so that no int sum can overflow
    int t_tot;
    block256_exclusive_scan(static_cast<int>(t & 0xffff), sh.scan, &t_tot);
    const int64_t t_lo = t_tot;
    block256_exclusive_scan(static_cast<int>(t >> 16), sh.scan, &t_tot);
    const int64_t total_cost = t_lo + (static_cast<int64_t>(t_tot) << 16);
    cost_a = total_cost * blockIdx.x / gridDim.x;
    cost_b = total_cost * (blockIdx.x + 1) / gridDim.x;
    if (tid == 0) {
      sh.rng[0] = items;
      sh.rng[1] = -1;
    }
    int64_t carry = 0;
    for (int base = 0; base < items && carry < cost_b; base += kBlockThreads) {
      const int i = base + tid;
      const int c = item_cost(i < items ? bk.counts[i] : 0);
      int tot;
      const int64_t p = carry + block256_exclusive_scan(c, sh.scan, &tot);
      if (c > 0 && p <= cost_a && cost_a < p + c) {
        sh.rng[0] = i;
        sh.rng[2] = static_cast<int>(cost_a - p);
      }
      if (c > 0 && p < cost_b && cost_b <= p + c) {
        sh.rng[1] = i;
        sh.rng[3] = static_cast<int>(cost_b - p);
      }
      carry += tot;
    }
    __syncthreads();
    it_begin = (cost_a < cost_b) ? sh.rng[0] : items;
    it_stop = (cost_a < cost_b) ? sh.rng[1] + 1 : items;
    it_step = 1;
    p_first = sh.rng[2];  // the range starts this far into its first item
    p_last = sh.rng[3];   // and ends this far into its last
  }

  for (int item = it_begin; item < it_stop; item += it_step) {
    // entries [e_lo, e_hi) of the item (in row order) are this workgroup's:
    // of an item's cost units the first kItemCost carry no entry
    const int e_lo = (bk.counts && item == it_begin) ? static_cast<int>(max<int64_t>(p_first - kItemCost, 0)) : 0;
    const int e_hi = (bk.counts && item == it_stop - 1) ? static_cast<int>(max<int64_t>(p_last - kItemCost, 0))
                                                         : 0x7fffffff;
    if (e_lo >= e_hi) continue;
    if (bk.counts && bk.counts[item] == 0) continue;  // no row chose it
    const int r = item / bk.nbmax, blk = item - r * bk.nbmax;
    const int L = clampi(bk.seq_lens[r], 0, bk.len_cap);
    const int q0 = clampi(bk.cu_q[r], 0, a.num_rows), q1 = clampi(bk.cu_q[r + 1], q0, a.num_rows);
    if (blk * kPage >= L || q1 <= q0) continue;
    const int pos0 = L - (q1 - q0);  // absolute position of the request's first row
    const int page = clampi(a.block_table[static_cast<size_t>(r) * a.ld_bt + blk], 0, pmax);
    const int nreq = min(kPage, L - blk * kPage);  // tokens of the block the request holds
    const int word = blk >> 5, bit = blk & 31;
    bool staged = false;

    // The rows of r that selected the block, kRowChunk rows at a time: the
    // top-k step left each row's selection as bit words (block b is bit b%32
    // of word b/32) with the count of selected blocks below each word, so one
    // 8-byte load per row gives both whether the row selected the block and
    // the block's rank in the row's selection. Row i of a pass is held by
    // thread i % 256 (segment i / 256); each wave's ballot per segment and
    // the 16 (segment, wave) counts in LDS number the hits in row order.
    constexpr int kSeg = kRowChunk / kBlockThreads;
    const uint64_t below = (1ull << lane) - 1ull;
    int carry = 0;  // entries of the item in earlier passes
    for (int c0 = q0; c0 < q1 && carry < e_hi; c0 += kRowChunk) {
      const int nc = min(kRowChunk, q1 - c0);
      uint64_t wd[kSeg], hits[kSeg];
#pragma unroll
      for (int k = 0; k < kSeg; ++k) {
        const int n = c0 + min(tid + kBlockThreads * k, nc - 1);
        wd[k] = bk.row_words[static_cast<size_t>(n) * bk.row_words_ld + word];
      }
#pragma unroll
      for (int k = 0; k < kSeg; ++k) {
        hits[k] = __ballot(tid + kBlockThreads * k < nc && ((static_cast<uint32_t>(wd[k]) >> bit) & 1u));
        if (lane == 0) sh.pcnt[k][wave] = __popcll(hits[k]);
      }
      // (this barrier also ends every wave's use of the previous pass's
      // entries and of the staged block)
      __syncthreads();
      int pre[kSeg], tot = 0;
#pragma unroll
      for (int k = 0; k < kSeg; ++k)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if (w == wave) pre[k] = tot;
          tot += sh.pcnt[k][w];
        }
      const int keep_lo = max(e_lo, carry), keep_hi = min(e_hi, carry + tot);
#pragma unroll
      for (int k = 0; k < kSeg; ++k) {
        const int idx = carry + pre[k] + __popcll(hits[k] & below);
        if (((hits[k] >> lane) & 1ull) && idx >= keep_lo && idx < keep_hi) {
          const uint32_t lo = static_cast<uint32_t>(wd[k]), hi = static_cast<uint32_t>(wd[k] >> 32);
          const int rank = static_cast<int>(hi) + __popc(lo & ((1u << bit) - 1u));
          sh.ent[idx - keep_lo] =
              static_cast<int>((c0 - q0 + tid + kBlockThreads * k) | (min(rank, kListRankMax) << kListRankShift));
        }
      }
      carry += tot;
      __syncthreads();
      const int total = max(keep_hi - keep_lo, 0);
      if (total == 0) continue;
      if (!staged) {  // the block's K and V, once per item, only when some row selected it
        staged = true;
        {
          // 16-byte pieces of the stored planes: 32 KiB of bf16 or 16 KiB of codes
          constexpr int kSrcPlane = kPage * kDim * (KV_FP8 ? 1 : 2);
          constexpr int kPieces = kSrcPlane / 16 / kBlockThreads;  // 8 or 4
          const u32x4* kg = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.k_cache) +
                                                           static_cast<size_t>(page) * kSrcPlane);
          const u32x4* vg = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.v_cache) +
                                                           static_cast<size_t>(page) * kSrcPlane);
          u32x4 kr[kPieces], vr[kPieces];
          uint32_t vabs = 0u;  // largest |V| as bf16 magnitude bits (order-preserving)
#pragma unroll
          for (int i = 0; i < kPieces; ++i) {
            kr[i] = __builtin_nontemporal_load(kg + tid + kBlockThreads * i);
            vr[i] = __builtin_nontemporal_load(vg + tid + kBlockThreads * i);
          }
          if constexpr (SCALE_MODE == 2) {
            if (tid < kPage) {
              sh.ks[tid] = a.k_scale[static_cast<size_t>(page) * kPage + tid];
              sh.vs[tid] = (tid < nreq) ? a.v_scale[static_cast<size_t>(page) * kPage + tid] : 0.f;
            }
          }
          u32x4* kd = reinterpret_cast<u32x4*>(sh.k);
          u32x4* vd = reinterpret_cast<u32x4*>(sh.v);
#pragma unroll
          for (int i = 0; i < kPieces; ++i) {
            const int q = tid + kBlockThreads * i;
            if constexpr (KV_FP8 != 0) {  // 16 codes -> 16 bf16 values (exact), same element order
              auto widen16 = [](u32x4 w, u32x4& lo, u32x4& hi) {
                const u32x2 a0 = fp8x4_to_bf16x4(w.x), a1 = fp8x4_to_bf16x4(w.y);
                const u32x2 a2 = fp8x4_to_bf16x4(w.z), a3 = fp8x4_to_bf16x4(w.w);
                lo = u32x4{a0.x, a0.y, a1.x, a1.y};
                hi = u32x4{a2.x, a2.y, a3.x, a3.y};
              };
              u32x4 lo, hi;
              widen16(kr[i], lo, hi);
              kd[2 * q] = lo;
              kd[2 * q + 1] = hi;
              widen16(vr[i], lo, hi);
              if (nreq < kPage) {  // slots past the request's last token can hold anything
                const int t0 = (q >> 7) * kSub;  // first token of the row's sub-page
                uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                  if (t0 + 2 * u >= nreq) w[u] &= 0xffff0000u;
                  if (t0 + 2 * u + 1 >= nreq) w[u] &= 0x0000ffffu;
                }
                lo = u32x4{w[0], w[1], w[2], w[3]};
                hi = u32x4{w[4], w[5], w[6], w[7]};
              }
              // a whole dim (16 tokens): token group p of the stored row is
              // group p ^ f of the dim
              const int f = v_swz(q);
              const u32x2 c0 = {lo.x, lo.y}, c1 = {lo.z, lo.w}, c2 = {hi.x, hi.y}, c3 = {hi.z, hi.w};
              const u32x2 t0 = (f & 1) ? c1 : c0, t1 = (f & 1) ? c0 : c1;
              const u32x2 t2 = (f & 1) ? c3 : c2, t3 = (f & 1) ? c2 : c3;
              const u32x2 o0 = (f & 2) ? t2 : t0, o1 = (f & 2) ? t3 : t1;
              const u32x2 o2 = (f & 2) ? t0 : t2, o3 = (f & 2) ? t1 : t3;
              const int vrow = v_row(q >> 7, q & (kDim - 1));
              vd[2 * vrow] = u32x4{o0.x, o0.y, o1.x, o1.y};
              vd[2 * vrow + 1] = u32x4{o2.x, o2.y, o3.x, o3.y};
              asm volatile("" ::: "memory");  // one piece at a time (fewer live registers)
            } else {
              kd[q] = kr[i];
              // half hh of dim row q/2 (groups 2hh, 2hh+1) goes to half
              // hh ^ (f >> 1) of the row, its two groups swapped when f & 1
              const int f = v_swz(q >> 1);
              u32x4 w = vr[i];
              if (nreq < kPage) {  // slots past the request's last token can hold anything
                const int t0 = (q >> 8) * kSub + 8 * (q & 1);  // first token of the piece
                uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                  if (t0 + 2 * u >= nreq) x[u] &= 0xffff0000u;
                  if (t0 + 2 * u + 1 >= nreq) x[u] &= 0x0000ffffu;
                }
                w = u32x4{x[0], x[1], x[2], x[3]};
              }
              vd[2 * v_row(q >> 8, (q >> 1) & (kDim - 1)) + ((q & 1) ^ (f >> 1))] =
                  (f & 1) ? u32x4{w.z, w.w, w.x, w.y} : w;
              if constexpr (SCALE_MODE == 0) {
                const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) vabs = max(vabs, max(x[u] & 0x7fffu, (x[u] >> 16) & 0x7fffu));
              }
            }
          }
          if constexpr (SCALE_MODE == 0) {
            vabs = wave_extreme_u32<true>(vabs);
            if (lane == 0) sh.vmax[wave] = vabs;
          }
        }
        __syncthreads();
      }
      // bf16 V with no scales: one power of two for all of the block's
      // partials, 2^ex > 128 max|V| >= |sum_t p_t v_t| (p_t <= 1), folded
      // into the softmax max, so the accumulators come out of the products
      // already scaled for fp16
      int blk_ex = 0;
      if constexpr (SCALE_MODE == 0) {
        const uint32_t vmb = max(max(sh.vmax[0], sh.vmax[1]), max(sh.vmax[2], sh.vmax[3]));
        if (vmb != 0u)
          blk_ex = clampi(__builtin_amdgcn_frexp_expf(__uint_as_float(vmb << 16)) + 7, -kHalfExpRange, kHalfExpRange);
      }
      // each wave takes every fourth (row, head group)
      const int nent = total * a.num_hgroups;
      auto entry_q = [&](int e, bf16x8 (&qv)[4]) {
        const int ee = min(e, max(nent - 1, 0));
        const int rl = min(static_cast<int>(static_cast<uint32_t>(sh.ent[ee / a.num_hgroups]) & kListRowMask),
                           q1 - q0 - 1);
        load_q_any(a, q0 + rl, ee % a.num_hgroups, qv);
      };
      // The query of the next entry is requested before the current entry's
      // products and its partial stores, and every entry issues the same
      // loads and stores, so the wait for that query leaves the stores in
      // flight. The first entry is peeled off so that the loop is entered with
      // the counters in the same state as from its own back edge.
      bf16x8 qa[4], qb[4];
      auto do_entry = [&](int e, const bf16x8 (&qv)[4]) {
        const uint32_t ent = static_cast<uint32_t>(sh.ent[e / a.num_hgroups]);
        const int rloc = min(static_cast<int>(ent & kListRowMask), q1 - q0 - 1);
        const int row = q0 + rloc, rank = min(static_cast<int>(ent >> kListRankShift), bk.topk - 1);
        const int hgi = e - (e / a.num_hgroups) * a.num_hgroups;
        const int vis = pos0 + rloc + 1;  // keys the row sees
        const int nval = clampi(vis - blk * kPage, 1, kPage);  // tokens of this block it sees
        // pass 1: the block's 128 logits (S^T per sub-page: token rows, head
        // columns) and their max, two sub-pages at a time with their two
        // product chains interleaved; the empty asm keeps the compiler from
        // pulling every sub-page's LDS operands into registers at once
        // (the row sees the whole block in all but its last selected block:
        // that case is compiled without the per-token visibility selects)
        float z[8][4];
        float mloc = -INFINITY;
        auto pass1 = [&](auto whole) {
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            bf16x8 ka[4], kb[4];
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
              ka[kc] = lds_k_op(sh, i, kc, lane);
              kb[kc] = lds_k_op(sh, i + 1, kc, lane);
            }
            f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
              sa = mfma_16x16x32(ka[kc], qv[kc], sa);
              sb = mfma_16x16x32(kb[kc], qv[kc], sb);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int ta = i * kSub + tok0 + t, tb = ta + kSub;
              const float za = sa[t] * zscale * ((SCALE_MODE == 2) ? sh.ks[ta] : 1.f);
              const float zb = sb[t] * zscale * ((SCALE_MODE == 2) ? sh.ks[tb] : 1.f);
              z[i][t] = (decltype(whole)::value || ta < nval) ? za : -INFINITY;
              z[i + 1][t] = (decltype(whole)::value || tb < nval) ? zb : -INFINITY;
              mloc = fmaxf(mloc, fmaxf(z[i][t], z[i + 1][t]));
            }
            asm volatile("" ::: "memory");
          }
        };
        if (nval == kPage)
          pass1(std::true_type{});
        else
          pass1(std::false_type{});
        const float m = max_across_rows(mloc);  // finite: token 0 is visible
        const float mb = m + static_cast<float>(blk_ex);
        // pass 2: probabilities and O^T += V^T P^T per sub-page
        float lsum = 0.f;
        f32x4 o[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // two sub-pages per 16x16x32 product: K index 8g+j of lane group g
        // is token 4g+j of the first sub-page for j < 4 and token 4g+j-4 of
        // the second for j >= 4, in the V operand and the probabilities alike
        i16x4 vreg[2][2][8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) vreg[0][h][dt] = lds_v_op(sh, h, dt, lane);
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const int b = (i >> 1) & 1;
          if (i + 2 < 8) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int dt = 0; dt < 8; ++dt) vreg[b ^ 1][h][dt] = lds_v_op(sh, i + 2 + h, dt, lane);
          }
          float e[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int tok = (i + (j >> 2)) * kSub + tok0 + (j & 3);
            e[j] = fast_exp2(z[i + (j >> 2)][j & 3] - mb);
            lsum += e[j];
            if constexpr (SCALE_MODE == 2) e[j] *= sh.vs[tok];
          }
          const bf16x8 p = __builtin_bit_cast(bf16x8, (u32x4{pk_bf16(e[0], e[1]), pk_bf16(e[2], e[3]),
                                                             pk_bf16(e[4], e[5]), pk_bf16(e[6], e[7])}));
          // tokens the row does not see have p = 0 and finite values (slots
          // past the request's last token were zeroed when staged)
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            const u32x2 w0 = __builtin_bit_cast(u32x2, vreg[b][0][dt]), w1 = __builtin_bit_cast(u32x2, vreg[b][1][dt]);
            o[dt] = mfma_16x16x32(__builtin_bit_cast(bf16x8, (u32x4{w0.x, w0.y, w1.x, w1.y})), p, o[dt]);
          }
          asm volatile("" ::: "memory");
        }
        const float l = sum_across_rows(lsum);
        // the block's partial in the row's slot for the block's rank, the
        // accumulator in fp16: a scalar V scale is folded in, then the head's
        // accumulator is scaled by 2^-e so that its largest magnitude is below
        // 1, and e is folded into the log2-domain max and the sum
        // (2^(m+e) * l*2^-e = 2^m * l), so the merge weighs the slots exactly
        // as it weighs fp32 partials. For bf16 V with no scales e is the
        // block's (chosen when it was staged) and the probabilities already
        // carry 2^-e, so the products come out scaled. Every path stores the same instructions
        // (the four lanes of a head store the same m and l), so the wait for
        // the next entry's query never has to wait for these stores.
        const int head = lane & 15;
        float* part = a.partials + ((static_cast<size_t>(row) * a.num_hgroups + hgi) * a.nsplit + rank) * kHalfPartStride;
        uint32_t* acc = reinterpret_cast<uint32_t*>(part + 2 * kHeadTile) + (head * kDim + tok0) / 2;
        if constexpr (SCALE_MODE == 0) {  // already scaled by 2^-blk_ex
          part[head] = mb;
          part[kHeadTile + head] = l;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
            *reinterpret_cast<u32x2*>(acc + dt * 8) = u32x2{pk_f16(o[dt][0], o[dt][1]), pk_f16(o[dt][2], o[dt][3])};
          return;
        }
        float mx = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int t = 0; t < 4; ++t) mx = fmaxf(mx, fabsf(o[dt][t]));
        mx = max_across_rows(mx) * fabsf(vscal);
        const int ex = (mx > 0.f) ? clampi(__builtin_amdgcn_frexp_expf(mx), -kHalfExpRange, kHalfExpRange) : 0;
        const float f = ldexpf(vscal, -ex);
        part[head] = m + static_cast<float>(ex);
        part[kHeadTile + head] = ldexpf(l, -ex);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *reinterpret_cast<u32x2*>(acc + dt * 8) = u32x2{pk_f16(o[dt][0] * f, o[dt][1] * f), pk_f16(o[dt][2] * f, o[dt][3] * f)};
      };
      if (wave < nent) {
        // two query buffers in turn (no register copies, which would wait
        // for the loads early)
        entry_q(wave, qa);
        entry_q(wave + 4, qb);  // clamped to the last entry: always issued
        do_entry(wave, qa);
        for (int e = wave + 4; e < nent; e += 8) {
          entry_q(e + 4, qa);
          do_entry(e, qb);
          if (e + 4 >= nent) break;
          entry_q(e + 8, qb);
          do_entry(e + 4, qa);
        }
      }
    }
  }
}

// Rows of each request that selected each of its blocks: workgroup (r, w)
// counts, over the rows of request r, the bits of selection word w. Each of
// its 16 waves takes 64 rows at a time (a 4096-row prefill request is one
// batch of four groups a wave; 4 waves took 11.8 us on a step of 8198 rows,
// 16 take 6.7) and counts each bit with one ballot (lane b keeps bit b's
// count), so no two lanes ever add to one counter. Every item's count is
// written (zeros too), so nothing needs clearing.
constexpr int kCountThreads = 1024;
constexpr int kCountWaves = kCountThreads / 64;

__global__ __launch_bounds__(kCountThreads) void msa_block_count_kernel(MsaBlockArgs bk, int num_rows) {
  __shared__ int s_cnt[kCountWaves][32];
  const int r = blockIdx.x, w = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q0 = clampi(bk.cu_q[r], 0, num_rows), q1 = clampi(bk.cu_q[r + 1], q0, num_rows);
  int acc = 0;
  constexpr int kBatch = 4;  // 64-row groups per wave requested at once
  for (int n0 = q0 + 64 * wave; n0 < q1; n0 += kBatch * kCountThreads) {
    uint32_t bits[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int n = n0 + j * kCountThreads + lane;
      bits[j] = static_cast<uint32_t>(bk.row_words[static_cast<size_t>(min(n, q1 - 1)) * bk.row_words_ld + w]);
      if (n >= q1) bits[j] = 0u;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      // groups with no selected block need no ballots
      const uint64_t m = __ballot(bits[j] != 0u);
      if (m == 0ull) continue;
#pragma unroll
      for (int b = 0; b < 32; ++b) {
        const int c = __popcll(__ballot((bits[j] >> b) & 1u));
        acc += (lane == b) ? c : 0;
      }
    }
  }
  if (lane < 32) s_cnt[wave][lane] = acc;
  __syncthreads();
  const int b = 32 * w + static_cast<int>(threadIdx.x);
  if (threadIdx.x < 32 && b < bk.nbmax) {
    int t = 0;
#pragma unroll
    for (int v = 0; v < kCountWaves; ++v) t += s_cnt[v][threadIdx.x];
    bk.counts[static_cast<size_t>(r) * bk.nbmax + b] = t;
  }
}

template <int KV_FP8, int SCALE_MODE>
hipError_t launch(const MsaAttnArgs& a, hipStream_t s) {
  const int64_t grid = static_cast<int64_t>(a.num_rows) * a.num_hgroups * a.nsplit;
  if (a.scores) {
    const int nbmax = min(min(a.ld_s, a.ld_bt), kMaxBlocksPerRow);
    // short rows: each wave selects alone (4 keys per lane, no barrier);
    // up to 1024 blocks the four waves share the work; longer rows again
    // wave by wave with 16 keys per lane and the rest re-read from memory
    if (nbmax <= 256)
      hipLaunchKernelGGL((msa_attn_select_kernel<KV_FP8, SCALE_MODE, 4>), dim3(static_cast<unsigned>(grid)),
                         dim3(kAttnThreads), 0, s, a);
    else if (nbmax <= 1024)
      hipLaunchKernelGGL((msa_attn_coop_kernel<KV_FP8, SCALE_MODE, 4>), dim3(static_cast<unsigned>(grid)),
                         dim3(kAttnThreads), 0, s, a);
    else
      hipLaunchKernelGGL((msa_attn_select_kernel<KV_FP8, SCALE_MODE, 16>), dim3(static_cast<unsigned>(grid)),
                         dim3(kAttnThreads), 0, s, a);
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

hipError_t msa_launch_block_count(const MsaBlockArgs& b, int num_rows, hipStream_t s) {
  hipLaunchKernelGGL(msa_block_count_kernel, dim3(static_cast<unsigned>(b.num_reqs), static_cast<unsigned>(b.row_words_ld)),
                     dim3(kCountThreads), 0, s, b, num_rows);
  return hipGetLastError();
}

hipError_t msa_launch_attn_block(const MsaAttnArgs& a, const MsaBlockArgs& b, int kv_dtype, int scale_mode,
                                 int num_wgs, hipStream_t s) {
  const dim3 g(static_cast<unsigned>(num_wgs)), t(kBlockThreads);
  if (kv_dtype == 0) {
    if (scale_mode == 0) hipLaunchKernelGGL((msa_attn_block_kernel<0, 0>), g, t, 0, s, a, b);
    else if (scale_mode == 1) hipLaunchKernelGGL((msa_attn_block_kernel<0, 1>), g, t, 0, s, a, b);
    else hipLaunchKernelGGL((msa_attn_block_kernel<0, 2>), g, t, 0, s, a, b);
  } else {
    if (scale_mode == 1) hipLaunchKernelGGL((msa_attn_block_kernel<1, 1>), g, t, 0, s, a, b);
    else hipLaunchKernelGGL((msa_attn_block_kernel<1, 2>), g, t, 0, s, a, b);
  }
  return hipGetLastError();
}

hipError_t msa_launch_merge(const MsaAttnArgs& a, hipStream_t s) {
  if (a.nsplit <= 1 && !a.half_partials) return hipSuccess;  // block partials: always merged, one slot too
  // (every split partial is in the fp16 slot format)
  const int64_t grid = (static_cast<int64_t>(a.num_rows) + 7) / 8 * 8 * a.num_q_heads;
  const int32_t* ctxp = a.scores ? static_cast<const int32_t*>(a.ctx_out) : a.ctx_in;
  if (a.half_partials)
    hipLaunchKernelGGL(msa_merge_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(kMergeThreads), 0, s, a, ctxp);
  else
    hipLaunchKernelGGL(msa_merge_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(kMergeThreads), 0, s, a, ctxp);
  return hipGetLastError();
}

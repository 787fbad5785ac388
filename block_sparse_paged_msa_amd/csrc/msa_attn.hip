// Sparse paged attention over a page-16 block table with an online softmax
// (vLLM PR #47287 page, 功能与动机: attention over the few logical blocks the
// indexer selected; 实现拆解 item 2: FP8 K/V with k_scale / v_scale, scalar or
// per-token-head; 实现拆解 item 3: paged attention on the page-16 view of the
// page-128 cache).
//
// Workgroup = (row, group of 16 query heads, split of split_tok tokens), four
// waves that each walk a contiguous run of 16-token sub-pages:
//   S^T[token][head] = K_sub (16x128) . Q^T (128x16)   v_mfma_f32_16x16x32_bf16
//   O^T[dim][head]  += V_sub^T (128x16) . P^T (16x16)  v_mfma_f32_16x16x16_bf16
// The S^T output layout (lane = head, four tokens per lane) is exactly the
// P^T operand layout of the second product, and V sub-pages are stored
// dim-major so each lane reads its four tokens of one dim as 8 contiguous
// bytes. FP8 codes are widened to bf16 in registers (exact); a per-token K
// scale multiplies the logit, a per-token V scale multiplies the probability
// fed to the PV product; scalar scales fold into the logit scale and the final
// normalisation. The four waves merge through LDS; splits of one row merge in
// the last-arriving workgroup (log2-domain LSE weights), so the result does
// not depend on arrival order.
#include "msa_internal.h"

using namespace msa;

namespace {

constexpr int kAttnThreads = 256;
constexpr int kPartStride = 2 * kHeadTile + kHeadTile * kDim;  // m[16], l[16], acc[16][128]

template <int KV_FP8>
__device__ __forceinline__ void load_k(const void* cache, int sub, int lane, bf16x8 (&ka)[4]) {
  if constexpr (!KV_FP8) {
    const uint16_t* kp = static_cast<const uint16_t*>(cache) + static_cast<size_t>(sub) * (kSub * kDim) +
                         (lane & 15) * kDim + (lane >> 4) * 8;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) ka[kc] = *reinterpret_cast<const bf16x8*>(kp + kc * 32);
  } else {
    const uint8_t* kp = static_cast<const uint8_t*>(cache) + static_cast<size_t>(sub) * (kSub * kDim) +
                        (lane & 15) * kDim + (lane >> 4) * 8;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(kp + kc * 32);
      const u32x2 lo = fp8x4_to_bf16x4(w.x), hi = fp8x4_to_bf16x4(w.y);
      ka[kc] = __builtin_bit_cast(bf16x8, (u32x4{lo.x, lo.y, hi.x, hi.y}));
    }
  }
}

template <int KV_FP8>
__device__ __forceinline__ void load_v(const void* cache, int sub, int lane, i16x4 (&va)[8]) {
  if constexpr (!KV_FP8) {
    const uint16_t* vp = static_cast<const uint16_t*>(cache) + static_cast<size_t>(sub) * (kDim * kSub) +
                         (lane & 15) * kSub + (lane >> 4) * 4;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) va[dt] = *reinterpret_cast<const i16x4*>(vp + dt * 16 * kSub);
  } else {
    const uint8_t* vp = static_cast<const uint8_t*>(cache) + static_cast<size_t>(sub) * (kDim * kSub) +
                        (lane & 15) * kSub + (lane >> 4) * 4;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      va[dt] = __builtin_bit_cast(i16x4, fp8x4_to_bf16x4(*reinterpret_cast<const uint32_t*>(vp + dt * 16 * kSub)));
  }
}

template <int KV_FP8, int SCALE_MODE>
__global__ __launch_bounds__(kAttnThreads) void msa_attn_kernel(MsaAttnArgs a) {
  __shared__ float s_m[4][kHeadTile];
  __shared__ float s_l[4][kHeadTile];
  __shared__ float s_o[4][kDim][kHeadTile + 1];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x % a.nsplit;
  const int rest = blockIdx.x / a.nsplit;
  const int hgi = rest % a.num_hgroups;
  const int n = rest / a.num_hgroups;
  const int ctx = clampi(a.ctx[n], 0, min(a.max_ctx, kSub * a.ld_table));
  const int nsplit_n = (ctx + a.split_tok - 1) / a.split_tok;
  const int nheads = min(kHeadTile, a.num_q_heads - hgi * kHeadTile);
  uint16_t* orow = a.out + (static_cast<size_t>(n) * a.num_q_heads + hgi * kHeadTile) * kDim;

  if (ctx == 0) {  // nothing selected: zeros
    if (split == 0)
      for (int i = tid; i < nheads * kDim; i += kAttnThreads) orow[i] = 0;
    return;
  }
  if (split >= nsplit_n) return;

  float kscal = 1.f, vscal = 1.f;
  if constexpr (SCALE_MODE == 1) {
    kscal = a.k_scale[0];
    vscal = a.v_scale[0];
  }
  const float zscale = a.scale_log2 * kscal;

  // Q^T as the B operand: column = head lane%16, K entries = dims kc*32 + 8*(lane/16)..
  const int h = lane & 15;
  bf16x8 qb[4];
  if (h < nheads) {
    const uint16_t* qp = a.q + (static_cast<size_t>(n) * a.num_q_heads + hgi * kHeadTile + h) * kDim + (lane >> 4) * 8;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qb[kc] = *reinterpret_cast<const bf16x8*>(qp + kc * 32);
  } else {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qb[kc] = bf16x8{};
  }

  const int sp_per_wave = a.split_tok / (4 * kSub);
  const int sp_begin = split * (a.split_tok / kSub) + wave * sp_per_wave;
  const int sp_end = min(sp_begin + sp_per_wave, (ctx + kSub - 1) / kSub);
  const int32_t* trow = a.table + static_cast<size_t>(n) * a.ld_table;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int sp = sp_begin; sp < sp_end; ++sp) {
    const int sub = clampi(trow[sp], 0, a.num_subpages - 1);
    const int nval = min(kSub, ctx - sp * kSub);
    bf16x8 ka[4];
    i16x4 va[8];
    load_k<KV_FP8>(a.k_cache, sub, lane, ka);
    load_v<KV_FP8>(a.v_cache, sub, lane, va);
    f32x4 ks4 = {1.f, 1.f, 1.f, 1.f}, vs4 = {1.f, 1.f, 1.f, 1.f};
    if constexpr (SCALE_MODE == 2) {
      ks4 = *reinterpret_cast<const f32x4*>(a.k_scale + static_cast<size_t>(sub) * kSub + (lane >> 4) * 4);
      vs4 = *reinterpret_cast<const f32x4*>(a.v_scale + static_cast<size_t>(sub) * kSub + (lane >> 4) * 4);
    }

    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) s = mfma_16x16x32(ka[kc], qb[kc], s);

    float z[4], mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 4 * (lane >> 4) + i;
      z[i] = (tok < nval) ? s[i] * zscale * ks4[i] : -INFINITY;
      mloc = fmaxf(mloc, z[i]);
    }
    const float m_new = fmaxf(m_run, max_across_rows(mloc));
    const float alpha = fast_exp2(m_run - m_new);
    float psum = 0.f;
    i16x4 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(z[i] - m_new);
      psum += p;
      pb[i] = static_cast<short>(f32_to_bf16(p * vs4[i]));
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = mfma_16x16x16(va[dt], pb, o[dt] * alpha);
  }

  // ---- merge the four waves through LDS ----
  const float l_w = sum_across_rows(l_run);
  if (lane < kHeadTile) {
    s_m[wave][lane] = m_run;
    s_l[wave][lane] = l_w;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[wave][dt * 16 + 4 * (lane >> 4) + i][lane & 15] = o[dt][i];
  __syncthreads();

  const int hh = tid & 15;
  const int d0 = tid >> 4;  // dims d0 + 16k
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][hh]);
  const float Ms = (M == -INFINITY) ? 0.f : M;
  float wt[4], Lsum = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wt[w] = (s_m[w][hh] == -INFINITY) ? 0.f : fast_exp2(s_m[w][hh] - Ms);
    Lsum += wt[w] * s_l[w][hh];
  }
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int d = d0 + 16 * k;
    acc[k] = wt[0] * s_o[0][d][hh] + wt[1] * s_o[1][d][hh] + wt[2] * s_o[2][d][hh] + wt[3] * s_o[3][d][hh];
  }

  if (nsplit_n == 1) {
    const float inv = (Lsum > 0.f) ? vscal / Lsum : 0.f;
    if (hh < nheads) {
#pragma unroll
      for (int k = 0; k < 8; ++k) orow[hh * kDim + d0 + 16 * k] = f32_to_bf16(acc[k] * inv);
    }
    return;
  }

  // ---- several splits: publish the partial, the last arriver merges ----
  const size_t slot0 = (static_cast<size_t>(n) * a.num_hgroups + hgi) * a.nsplit;
  float* part = a.partials + (slot0 + split) * kPartStride;
  if (tid < kHeadTile) {
    part[tid] = M;
    part[kHeadTile + tid] = Lsum;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) part[2 * kHeadTile + hh * kDim + d0 + 16 * k] = acc[k];
  __threadfence();
  __syncthreads();
  int32_t* counter = a.counters + static_cast<size_t>(n) * a.num_hgroups + hgi;
  if (tid == 0) s_last = (atomicAdd(counter, 1) == nsplit_n - 1) ? 1 : 0;
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  const float* base = a.partials + slot0 * kPartStride;
  float Mg = -INFINITY;
  for (int sidx = 0; sidx < nsplit_n; ++sidx) Mg = fmaxf(Mg, base[sidx * kPartStride + hh]);
  float Lg = 0.f, og[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int sidx = 0; sidx < nsplit_n; ++sidx) {
    const float* ps = base + sidx * kPartStride;
    const float w = fast_exp2(ps[hh] - Mg);
    Lg += w * ps[kHeadTile + hh];
#pragma unroll
    for (int k = 0; k < 8; ++k) og[k] += w * ps[2 * kHeadTile + hh * kDim + d0 + 16 * k];
  }
  const float inv = (Lg > 0.f) ? vscal / Lg : 0.f;
  if (hh < nheads) {
#pragma unroll
    for (int k = 0; k < 8; ++k) orow[hh * kDim + d0 + 16 * k] = f32_to_bf16(og[k] * inv);
  }
  if (tid == 0) atomicExch(counter, 0);  // leave the counter at zero for the next call
}

template <int KV_FP8, int SCALE_MODE>
hipError_t launch(const MsaAttnArgs& a, hipStream_t s) {
  const int64_t grid = static_cast<int64_t>(a.num_rows) * a.num_hgroups * a.nsplit;
  hipLaunchKernelGGL((msa_attn_kernel<KV_FP8, SCALE_MODE>), dim3(static_cast<unsigned>(grid)),
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

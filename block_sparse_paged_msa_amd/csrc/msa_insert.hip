// The step before the path: new tokens written into the paged caches (vLLM PR
// #47287 page, 实现拆解 items 1, 2 and 5: the fused K/V insert writes the
// separate K and V planes and, unless the layer reuses another layer's index,
// the index cache; FP8 caches carry per-token-head or scalar K/V scales).
//
// Sixteen lanes per new token, eight dims each of its K, V and index-K rows
// (one 16-byte load per row and lane, issued with the slot loads), so the
// lanes of one DPP row hold a token's whole row for its scale. K and index-K
// pieces go into their shuffled tiles as one contiguous 8-element run per
// lane; V is dim-major ([128 dims][16 token slots] per sub-page).
//
// Quantisation (each code decided in fp32): per-token-head scale
// s = max|x| / 448 over the token-head's 128 values (1 for an all-zero row),
// code = e4m3fn RNE of clamp(x / s, -448, 448); a scalar scale is read, not
// written; bf16 caches store bf16 RNE of x / s with s = 1 unless scalar.
// An FP8 index cache (the optional FP8 index storage named on the vLLM PR
// #54682 page, 相关 PRs) takes each token's index key by the per-token rule:
// s = max|x| / 448 over its 128 values, codes e4m3fn RNE of clamp(x / s).
#include "msa_kernels.h"

using namespace msa;

namespace {

constexpr int kInsertThreads = 256;
constexpr float kE4m3Max = 448.f;

struct alignas(16) f32x8 {
  float v[8];
};

__device__ __forceinline__ f32x8 widen(u32x4 w) {
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.v[2 * i] = __uint_as_float(w[i] << 16);
    r.v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
  return r;
}

// Scale of one token-head row given its largest magnitude.
__device__ __forceinline__ float row_scale(const MsaInsertArgs& a, int plane, float amax) {
  if (a.scale_mode == 1) return plane == 0 ? a.k_scale[0] : a.v_scale[0];
  if (a.scale_mode == 2 && a.kv_fp8) return amax > 0.f ? amax / kE4m3Max : 1.f;
  return 1.f;
}

__device__ __forceinline__ uint32_t fp8_code(float x, float s) {
  const float y = fminf(fmaxf(x / s, -kE4m3Max), kE4m3Max);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false)) & 0xffu;
}

// Eight values of one row held by a lane whose 16-lane DPP row holds the
// whole 128-value row: the row's per-token scale and the lane's eight codes.
__device__ __forceinline__ u32x2 fp8_row_codes(const f32x8& x, float& s) {
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x.v[e]));
  amax = max16(amax);
  s = amax > 0.f ? amax / kE4m3Max : 1.f;
  uint32_t code[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) code[e >> 2] |= fp8_code(x.v[e], s) << (8 * (e & 3));
  return u32x2{code[0], code[1]};
}

// One token whose workgroup's sixteen do not fill one sub-page in order
// (decode: scattered slots), written by the 16 lanes that hold its pieces (8
// dims each of its K, V and index-K rows, loaded with the slots): the K and
// index-K pieces as contiguous runs of their tiles, the V piece as 8 dim rows
// of the dim-major sub-page. The reductions run in every lane; a skipped slot
// only writes nothing.
__device__ __forceinline__ void insert_token(const MsaInsertArgs& a, int slot, u32x4 kw, u32x4 vw, u32x4 iw) {
  const int c = threadIdx.x & 15;
  const bool valid = slot >= 0 && (slot >> 7) < a.num_pages;  // else skipped (or outside the caches)
  const int page = slot >> 7, off = slot & (kPage - 1);
  const int sub = kSubsPerPage * page + (off >> 4), j = off & (kSub - 1);
  const size_t tile = static_cast<size_t>(sub) * (kSub * kDim);  // the sub-page (one KV head)
  if (a.index_k_new) {
    const size_t at = static_cast<size_t>(page) * (kPage * kDim) + (off >> 4) * (kSub * kDim) + (c * 16 + j) * 8;
    if (a.index_scale_out) {
      float s;
      const u32x2 codes = fp8_row_codes(widen(iw), s);
      if (valid) {
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(a.index_k) + at) = codes;
        if (c == 0) a.index_scale_out[static_cast<size_t>(page) * kPage + off] = s;
      }
    } else if (valid) {
      *reinterpret_cast<u32x4*>(a.index_k + at) = iw;
    }
  }
#pragma unroll
  for (int plane = 0; plane < 2; ++plane) {
    const f32x8 x = widen(plane == 0 ? kw : vw);
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x.v[e]));
    const float s = row_scale(a, plane, max16(amax));  // the 16 lanes hold the whole row
    if (!valid) continue;
    if (a.scale_mode == 2 && c == 0) (plane == 0 ? a.k_scale_out : a.v_scale_out)[static_cast<size_t>(sub) * kSub + j] = s;
    if (plane == 0) {  // dims 8c..8c+7 of token j: one run of the shuffled tile
      if (a.kv_fp8) {
        uint32_t code[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) code[e >> 2] |= fp8_code(x.v[e], s) << (8 * (e & 3));
        *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(a.k_cache) + tile + (c * 16 + j) * 8) = u32x2{code[0], code[1]};
      } else {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = f32_to_bf16(x.v[2 * i] / s) | (static_cast<uint32_t>(f32_to_bf16(x.v[2 * i + 1] / s)) << 16);
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.k_cache) + tile + (c * 16 + j) * 8) = w;
      }
    } else {  // dim rows 8c..8c+7 of the dim-major sub-page, slot j of each
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const size_t at = tile + static_cast<size_t>(8 * c + e) * kSub + j;
        if (a.kv_fp8)
          static_cast<uint8_t*>(a.v_cache)[at] = static_cast<uint8_t>(fp8_code(x.v[e], s));
        else
          static_cast<uint16_t*>(a.v_cache)[at] = f32_to_bf16(x.v[e] / s);
      }
    }
  }
}

// Sixteen tokens that fill one sub-page in order (a prefill chunk): the
// workgroup quantises them, lays the K / index-K tiles and the dim-major V
// sub-page out in LDS, and writes each as one contiguous run. Thread i takes
// token i/16 and dims 8*(i%16).. of it (kw, vw, iw: its K, V and index-K
// pieces, loaded by the caller), so the 16 lanes of a DPP row hold one
// token's whole row for the scale.
__device__ __forceinline__ void insert_subpage(const MsaInsertArgs& a, int slot0, uint8_t* lds, u32x4 kw, u32x4 vw,
                                               u32x4 iw) {
  const int tid = threadIdx.x, j = tid >> 4, c = tid & 15;
  const int page = slot0 >> 7, sub = kSubsPerPage * page + ((slot0 & (kPage - 1)) >> 4);
  const int nbytes = a.kv_fp8 ? 1 : 2;
  const int kv_bytes = kSub * kDim * nbytes;  // one plane of one sub-page
  uint8_t* ks = lds;                 // K tile
  uint8_t* vs = lds + kv_bytes;      // V sub-page
  uint16_t* is = reinterpret_cast<uint16_t*>(lds + 2 * kv_bytes);  // index-K tile
#pragma unroll
  for (int plane = 0; plane < 2; ++plane) {
    const f32x8 x = widen(plane == 0 ? kw : vw);
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x.v[e]));
    const float s = row_scale(a, plane, max16(amax));
    if (a.scale_mode == 2 && c == 0) (plane == 0 ? a.k_scale_out : a.v_scale_out)[static_cast<size_t>(sub) * kSub + j] = s;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // element (dim 8c+e, token j): tile slot (c*16 + j)*8 + e for K, dim row (8c+e)*16 + j for V
      const int at = plane == 0 ? (c * 16 + j) * 8 + e : (8 * c + e) * kSub + j;
      uint8_t* dst = plane == 0 ? ks : vs;
      if (a.kv_fp8)
        dst[at] = static_cast<uint8_t>(fp8_code(x.v[e], s));
      else
        reinterpret_cast<uint16_t*>(dst)[at] = f32_to_bf16(x.v[e] / s);
    }
  }
  if (a.index_k_new) {
    if (a.index_scale_out) {  // fp8 index: per-token scale over the DPP row holding token j
      float s;
      const u32x2 codes = fp8_row_codes(widen(iw), s);
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(is) + (c * 16 + j) * 8) = codes;
      if (c == 0) a.index_scale_out[static_cast<size_t>(page) * kPage + (slot0 & (kPage - 1)) + j] = s;
    } else {
      *reinterpret_cast<u32x4*>(is + (c * 16 + j) * 8) = iw;
    }
  }
  __syncthreads();
  // each plane of the sub-page as one contiguous run: 16 bytes per thread
  const int per = kv_bytes / 16;  // 16-byte pieces per plane (128 or 256)
  for (int i = tid; i < per; i += kInsertThreads) {
    reinterpret_cast<u32x4*>(static_cast<uint8_t*>(a.k_cache) + static_cast<size_t>(sub) * kv_bytes)[i] =
        reinterpret_cast<const u32x4*>(ks)[i];
    reinterpret_cast<u32x4*>(static_cast<uint8_t*>(a.v_cache) + static_cast<size_t>(sub) * kv_bytes)[i] =
        reinterpret_cast<const u32x4*>(vs)[i];
  }
  if (a.index_k_new) {
    // the index tile: 4 KiB of bf16 (256 pieces) or 2 KiB of codes (128)
    const int ibytes = a.index_scale_out ? 1 : 2;
    uint8_t* idst = reinterpret_cast<uint8_t*>(a.index_k) +
                    (static_cast<size_t>(page) * (kPage * kDim) + ((slot0 & (kPage - 1)) >> 4) * (kSub * kDim)) * ibytes;
    if (tid < kSub * kDim * ibytes / 16)
      reinterpret_cast<u32x4*>(idst)[tid] = reinterpret_cast<const u32x4*>(is)[tid];
  }
}

// Workgroup = 16 consecutive tokens, thread i holding 8 dims of token i/16's
// K, V and index-K rows. When their slots are one whole sub-page in order (a
// prefill chunk), the sub-page path writes it in contiguous runs; otherwise
// every token is written at its own slot by the 16 lanes that hold it.
__global__ __launch_bounds__(kInsertThreads) void msa_insert_kernel(MsaInsertArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[3 * kSub * kDim * 2];
  const int t0 = blockIdx.x * kSub;
  const int lt = threadIdx.x & 15;
  const int sl = t0 + lt < a.num_tokens ? a.slot_mapping[t0 + lt] : -1;
  // the sub-page path's pieces are requested with the slots, before the
  // path is known (one round trip instead of two); one KV head, so token t's
  // rows start at t * 128, and the token index is clamped to the last token
  const int tp = min(t0 + static_cast<int>(threadIdx.x >> 4), a.num_tokens - 1);
  const size_t po = static_cast<size_t>(tp) * kDim + 8 * lt;
  const u32x4 kw = *reinterpret_cast<const u32x4*>(a.k_new + po);
  const u32x4 vw = *reinterpret_cast<const u32x4*>(a.v_new + po);
  u32x4 iw = {0u, 0u, 0u, 0u};
  if (a.index_k_new) iw = *reinterpret_cast<const u32x4*>(a.index_k_new + po);
  const int slot0 = __shfl(sl, 0, 16);
  const bool whole = t0 + kSub <= a.num_tokens && slot0 >= 0 && (slot0 & (kSub - 1)) == 0 &&
                     (slot0 >> 7) < a.num_pages && a.num_kv_heads == 1;
  // every lane compares its token's slot (all four waves see the same 16)
  const bool in_order = __all(sl == slot0 + lt);
  if (__builtin_amdgcn_readfirstlane(whole && in_order)) {
    insert_subpage(a, slot0, lds, kw, vw, iw);
    return;
  }
  // lane group g of wave w: token t0 + 4w + g, whose slot lane 4w + g holds
  // (past the last token the slot is -1)
  insert_token(a, __shfl(sl, static_cast<int>(threadIdx.x >> 4) & 15), kw, vw, iw);
}

}  // namespace

hipError_t msa_launch_insert(const MsaInsertArgs& a, hipStream_t s) {
  const int grid = (a.num_tokens + kSub - 1) / kSub;
  hipLaunchKernelGGL(msa_insert_kernel, dim3(static_cast<unsigned>(grid)), dim3(kInsertThreads), 0, s, a);
  return hipGetLastError();
}

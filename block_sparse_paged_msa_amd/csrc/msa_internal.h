// Internal declarations shared by the library's HIP sources: vector types,
// number-format helpers, MFMA wrappers, wave/block reductions, and the
// metadata and index-score launchers that msa_api.hip calls (the top-k,
// attention and insert ones are in msa_kernels.h). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kPage = 128;        // tokens per page-128 page / sparse block
constexpr int kSub = 16;          // tokens per page-16 sub-page
constexpr int kSubsPerPage = 8;   // sub-pages per page
constexpr int kDim = 128;         // head dim and index dim
constexpr int kRowsPerUnit = 64;  // query rows of one request per score unit
constexpr int kHeadTile = 16;     // query heads per attention MFMA tile
constexpr int kMaxReqs = 4096;    // requests per batch (LDS-resident prefix)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Two floats -> two bf16 (round to nearest even, denormals kept, NaN stays a
// quiet NaN), low half first: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// float -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return static_cast<uint16_t>(pk_bf16(f, 0.f)); }


// Four e4m3fn codes (one dword) -> four bf16 values packed in two dwords.
// e4m3 values are exactly representable in bf16, so taking the top half of
// the exact fp32 conversion is exact.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  u32x2 r;
  r.x = __builtin_amdgcn_perm(__float_as_uint(lo.y), __float_as_uint(lo.x), 0x07060302u);
  r.y = __builtin_amdgcn_perm(__float_as_uint(hi.y), __float_as_uint(hi.x), 0x07060302u);
  return r;
}

// D = A(16x32) * B(32x16) + C; lane l supplies A row l%16 / B column l%16 and
// eight consecutive K entries selected by l/16; D lane l holds rows 4*(l/16)+i
// of column l%16.
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Same with K = 16: four K entries per lane.
__device__ __forceinline__ f32x4 mfma_16x16x16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Max over the 16 lanes of each DPP row, in every lane of the row: quad swaps,
// then half-row and row mirrors pair up the remaining groups.
__device__ __forceinline__ float max16(float v) {
  int x = __float_as_int(v);
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xf, 0xf, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xf, 0xf, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x141, 0xf, 0xf, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x140, 0xf, 0xf, false))));
  return __int_as_float(x);
}

// Lanes l, l^16, l^32, l^48 (the same lane of the four rows): gfx950's
// permlane swaps exchange rows 0<->1, 2<->3 and halves 0-31 <-> 32-63; with
// both operands equal, the two results hold the value and its partner.
__device__ __forceinline__ float max_across_rows(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

__device__ __forceinline__ float sum_across_rows(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;  // log2(e): natural-log logits to log2 domain
constexpr float kLn2 = 0.6931471805599453f;    // ln(2): back to natural log

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by
// 1, 2, 4, 8 inside each 16-lane row, then the row totals are carried forward
// (lane 15 into row 1 and row 3, then lane 31 into rows 2 and 3). Lanes whose
// source is outside the row or whose row is masked add the `old` value 0.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Exclusive prefix sum over a 256-thread block; `scratch` holds 4 ints.
__device__ __forceinline__ int block256_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_inclusive_scan(v);
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int t = scratch[w];
    base += (w < wave) ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

}  // namespace msa

// ---------------------------------------------------------------------------
// Kernel launchers (host functions defined next to each kernel).
// ---------------------------------------------------------------------------
struct MsaMetaArgs {
  const int32_t* seq_lens;
  const int32_t* query_lens;
  int32_t* cu_q;
  int32_t* cu_k;
  int32_t* cu_blocks;
  int32_t* cu_units;
  int32_t* row_req;
  int32_t* row_pos;
  int32_t num_reqs;
  int32_t num_rows;
  int32_t len_cap;     // seq_lens are clamped to [0, len_cap]
};
hipError_t msa_launch_meta(const MsaMetaArgs& a, hipStream_t s);

struct MsaScoreArgs {
  const uint16_t* index_q;
  const void* index_k;        // bf16 keys, or e4m3fn codes when index_scale is set
  const float* index_scale;   // [P][128] per-token scales of an fp8 index cache, or null
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* query_lens;
  float* scores;
  // batch metadata, written by workgroup 0 when write_meta != 0
  int32_t* cu_q;
  int32_t* cu_k;
  int32_t* cu_blocks;
  int32_t* cu_units;
  int32_t* row_req;
  int32_t* row_pos;
  int32_t ld_s;
  int32_t ld_bt;
  int32_t num_reqs;
  int32_t num_rows;
  int32_t num_pages;
  int32_t len_cap;
  int32_t blocks_per_req;  // host bound S on any request's blocks: slot r*S + j
  int32_t write_meta;
  int32_t skip_big;        // requests with more than 64 rows are left to the tile kernel
};
hipError_t msa_launch_score(const MsaScoreArgs& a, int num_wgs, hipStream_t s);
// Requests with more than 64 query rows: 512-row blocks x runs of 8 (or 16)
// index-K pages, one MFMA tile workgroup per item.
hipError_t msa_launch_score_tile(const MsaScoreArgs& a, int num_wgs, hipStream_t s);
int msa_score_tile_items_bound(int64_t num_rows, int64_t blocks_bound);

// Top-k block selection of one query row by a 256-thread workgroup (vLLM PR
// #54682 page, 实现拆解 item 1: the fused top-k keeps each row's highest-scoring
// blocks and also yields the row's context length).
//
// The row's block scores sit in LDS as order-preserving 32-bit keys. The
// K'-th largest key T is found by an MSB-first radix select (4 passes of 8
// bits with LDS histograms); every key above T is kept, and among keys equal
// to T the lowest block ids are kept until K' blocks are chosen. A block-wide
// prefix count over ascending block ids then gives each kept block its rank,
// so the caller receives the selection in ascending block-id order.
#pragma once

#include "msa_internal.h"

namespace msa {

constexpr int kSelectThreads = 256;
constexpr int kMaxBlocksPerRow = 8192;  // 2^20 tokens of context

// Larger float -> larger unsigned key; -0.0 maps to the key of +0.0.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct SelectLds {
  int hist[256];
  int scan[4];
  int digit;
  int need;
  int eq_total;
  int last_kept;
};

// Keeps K' = min(topk, nb) of the nb keys; calls emit(rank, block) for each
// kept block (ranks 0..K'-1 in ascending block order, any thread may emit).
// before_compaction() runs in every thread after the threshold is known and
// before the first emit(); emit(rank, block) runs in the thread that owns
// block = base + threadIdx.x of one 256-block chunk.
// Returns K'; *ctx_out gets sum over kept blocks of min(128, v - 128*block)
// in every thread: every block but the last (nb-1) holds 128 visible tokens,
// so the sum is 128*K' minus the last block's invisible tail when it is kept.
// All 256 threads must call it.
template <typename Emit, typename BeforeCompaction>
__device__ __forceinline__ int select_row(const uint32_t* keys, int nb, int topk, int v, SelectLds& sl, Emit emit,
                                          int* ctx_out, BeforeCompaction before_compaction) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kk = min(topk, nb);
  const bool partial = kk < nb;
  uint32_t T = 0;
  int need = 0, eq_total = 0;
  if (tid == 0) sl.last_kept = 0;
  if (partial) {
    sl.hist[tid] = 0;
    __syncthreads();
    uint32_t prefix = 0;
    need = kk;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int e = tid; e < nb; e += kSelectThreads) {
        const uint32_t k = keys[e];
        const bool match = (shift == 24) || ((k >> (shift + 8)) == (prefix >> (shift + 8)));
        if (match) atomicAdd(&sl.hist[(k >> shift) & 255u], 1);
      }
      __syncthreads();
      if (wave == 0) {
        // lane owns digits 255-4*lane .. 252-4*lane (descending); one wave scan
        int c[4], local = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c[i] = sl.hist[255 - 4 * lane - i];
          local += c[i];
        }
        const int incl = wave_inclusive_scan(local);
        int run = incl - local;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (run < need && need <= run + c[i]) {
            sl.digit = 255 - 4 * lane - i;
            sl.need = need - run;
            sl.eq_total = c[i];
          }
          run += c[i];
          sl.hist[255 - 4 * lane - i] = 0;  // ready for the next pass
        }
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(sl.digit) << shift;
      need = sl.need;
    }
    T = prefix;
    eq_total = sl.eq_total;  // keys equal to T (the last pass bins them exactly)
  }

  before_compaction();  // caller hook: per-thread data that emit() reads (same thread, no barrier)

  // every key equal to T is kept unless the tie straddles the cut
  const bool all_eq_kept = !partial || need == eq_total;
  int carry_eq = 0, carry_sel = 0;
  for (int base = 0; base < nb; base += kSelectThreads) {
    const int e = base + tid;
    const bool valid = e < nb;
    const uint32_t k = valid ? keys[e] : 0u;
    int keep;
    if (all_eq_kept) {
      keep = valid && (!partial || k >= T) ? 1 : 0;
    } else {
      const int eq = (valid && k == T) ? 1 : 0;
      int tot_eq;
      const int rank_eq = carry_eq + block256_exclusive_scan(eq, sl.scan, &tot_eq);
      keep = valid && (k > T || (eq && rank_eq < need)) ? 1 : 0;
      carry_eq += tot_eq;
    }
    int tot_sel;
    const int pos = carry_sel + block256_exclusive_scan(keep, sl.scan, &tot_sel);
    if (keep) {
      emit(pos, e);
      if (e == nb - 1) sl.last_kept = 1;
    }
    carry_sel += tot_sel;
  }
  __syncthreads();
  *ctx_out = kPage * kk - (sl.last_kept ? kPage * nb - v : 0);
  return kk;
}

// ---------------------------------------------------------------------------
// The same selection computed by one wave alone (every wave of a workgroup
// can run it on the same LDS keys and get the same answer with no
// workgroup barrier). hist: 256 ints of LDS private to the wave.
// ---------------------------------------------------------------------------
struct WaveSelection {
  uint32_t T;        // keep keys > T, and keys == T among the lowest ids
  int need;          // keys equal to T that are kept (lowest ids first)
  int kk;            // K' = min(topk, nb)
  bool partial;      // kk < nb
  bool all_eq_kept;  // every key >= T is kept
};

__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// The keys of blocks e = lane + 64*i, i < KR, in registers (0 past nb);
// blocks from 64*KR on are read from LDS when needed.
template <int KR>
struct WaveKeys {
  uint32_t k[KR];
};

template <int KR>
__device__ __forceinline__ void wave_load_keys(const uint32_t* keys, int nb, WaveKeys<KR>& wk) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < KR; ++i) wk.k[i] = (lane + 64 * i < nb) ? keys[lane + 64 * i] : 0u;
}

template <int KR>
__device__ __forceinline__ WaveSelection wave_select(const uint32_t* keys, const WaveKeys<KR>& wk, int nb, int topk,
                                                     int* hist) {
  const int lane = threadIdx.x & 63;
  WaveSelection w;
  w.kk = min(topk, nb);
  w.partial = w.kk < nb;
  w.T = 0;
  w.need = 0;
  w.all_eq_kept = true;
  if (!w.partial) return w;
  uint32_t prefix = 0;
  int need = w.kk;
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0;
    wave_lds_order();
    auto bin = [&](uint32_t k) {
      const bool match = (shift == 24) || ((k >> (shift + 8)) == (prefix >> (shift + 8)));
      if (match) atomicAdd(&hist[(k >> shift) & 255u], 1);
    };
#pragma unroll
    for (int i = 0; i < KR; ++i)
      if (lane + 64 * i < nb) bin(wk.k[i]);
    for (int e = lane + 64 * KR; e < nb; e += 64) bin(keys[e]);
    wave_lds_order();
    int c[4], local = 0;  // lane owns digits 255-4*lane .. 252-4*lane (descending)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = hist[255 - 4 * lane - i];
      local += c[i];
    }
    const int incl = wave_inclusive_scan(local);
    int run = incl - local, my_digit = 0, my_need = 0, my_cnt = 0;
    bool found = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (run < need && need <= run + c[i]) {
        found = true;
        my_digit = 255 - 4 * lane - i;
        my_need = need - run;
        my_cnt = c[i];
      }
      run += c[i];
    }
    // exactly one lane holds the digit: broadcast it with readlane
    const int src = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<unsigned long long>(__ballot(found))) - 1);
    prefix |= static_cast<uint32_t>(__builtin_amdgcn_readlane(my_digit, src)) << shift;
    need = __builtin_amdgcn_readlane(my_need, src);
    const int cnt = __builtin_amdgcn_readlane(my_cnt, src);
    wave_lds_order();
    if (need == cnt) {
      // every key sharing the prefix so far is kept: keys >= prefix (lower
      // bits zero) are exactly the K' largest, no tie straddles the cut
      w.T = prefix;
      w.need = 0;
      w.all_eq_kept = true;
      return w;
    }
  }
  w.T = prefix;
  w.need = need;
  w.all_eq_kept = false;  // keys equal to T straddle the cut: lowest ids first
  return w;
}

// Visits the kept blocks in ascending id order: visit(rank, block) in the
// lane that examined the block. Returns the context length
// 128*K' - (block nb-1 kept ? 128*nb - v : 0) in every lane.
template <int KR, typename Visit>
__device__ __forceinline__ int wave_compact(const uint32_t* keys, const WaveKeys<KR>& wk, int nb, int v,
                                            const WaveSelection& w, Visit visit) {
  const int lane = threadIdx.x & 63;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int carry = 0, carry_eq = 0;
  bool last_kept = false;
  auto step = [&](int e, uint32_t k) {
    const bool valid = e < nb;
    bool keep;
    if (!w.partial) {
      keep = valid;
    } else if (w.all_eq_kept) {
      keep = valid && k >= w.T;
    } else {
      const bool eq = valid && k == w.T;
      const unsigned long long em = __ballot(eq);
      const int rank_eq = carry_eq + __popcll(em & lt);
      carry_eq += __popcll(em);
      keep = valid && (k > w.T || (eq && rank_eq < w.need));
    }
    const unsigned long long km = __ballot(keep);
    if (keep) {
      visit(carry + __popcll(km & lt), e);
      if (e == nb - 1) last_kept = true;
    }
    carry += __popcll(km);
  };
#pragma unroll
  for (int i = 0; i < KR; ++i)
    if (64 * i < nb) step(lane + 64 * i, wk.k[i]);
  for (int base = 64 * KR; base < nb; base += 64) step(base + lane, base + lane < nb ? keys[base + lane] : 0u);
  const bool lk = __ballot(last_kept) != 0ull;
  return kPage * w.kk - (lk ? kPage * nb - v : 0);
}

}  // namespace msa

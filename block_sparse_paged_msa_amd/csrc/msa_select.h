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
        int incl = local;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o);
          if (lane >= o) incl += y;
        }
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

}  // namespace msa

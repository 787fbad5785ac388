// Top-k block selection of one query row (vLLM PR #54682 page, 实现拆解 item
// 1: the fused top-k keeps each row's highest-scoring blocks and also yields
// the row's context length).
//
// The row's block scores are order-preserving 32-bit keys. The K'-th largest
// key T is found by an MSB-first radix select with 8-bit digits and LDS
// histograms, its first window starting at the highest bit where the row's
// largest and smallest keys differ; every key above T is kept, and among
// keys equal to T the lowest block ids are kept until K' blocks are chosen.
// Prefix counts of the keep ballots over ascending block ids give each kept
// block its rank, so the selection comes out in ascending block-id order.
// Two forms: one wave selecting alone from keys in its registers
// (wave_select, wave_locate), and the four waves of a workgroup sharing one
// histogram per pass (coop_select, coop_locate).
#pragma once

#include "msa_kernels.h"

namespace msa {

constexpr int kSelectThreads = 256;
constexpr int kMaxBlocksPerRow = 8192;  // 2^20 tokens of context

// Larger float -> larger unsigned key; -0.0 maps to the key of +0.0.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---------------------------------------------------------------------------
// The selection computed by one wave alone, from keys held in registers
// (every wave of a workgroup can run it on the same row and get the same
// answer with no workgroup barrier). The bits above the highest bit where
// the largest and smallest keys differ are shared by every key, so the first
// 8-bit window starts at that bit; each pass has its own histogram in the
// wave's LDS, cleared once up front.
// ---------------------------------------------------------------------------
constexpr int kWaveRadixPasses = 4;

struct WaveSelection {
  uint32_t T;        // keep keys > T, and keys == T among the lowest ids
  int need;          // keys equal to T that are kept (lowest ids first)
  int kk;            // K' = min(topk, nb)
  bool partial;      // kk < nb
  bool all_eq_kept;  // every key >= T is kept
};

// The keys of blocks e = lane + 64*i, i < KR, in registers; slots at or
// past nb are ignored. Blocks from 64*KR on come from tail_key(e).
template <int KR>
struct WaveKeys {
  uint32_t k[KR];
};

__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Clears a wave's kWaveRadixPasses x 256 histogram counters.
__device__ __forceinline__ void wave_clear_hist(int (*hist)[256]) {
  const int lane = threadIdx.x & 63;
  i32x4* h = reinterpret_cast<i32x4*>(&hist[0][0]);
#pragma unroll
  for (int i = 0; i < kWaveRadixPasses; ++i) h[i * 64 + lane] = i32x4{0, 0, 0, 0};
}

// Max / min of an unsigned value over the wave, in every lane (DPP inside
// each 16-lane row, then the row and half swaps).
template <bool MAX>
__device__ __forceinline__ uint32_t wave_extreme_u32(uint32_t x) {
  auto op = [](uint32_t p, uint32_t q) { return MAX ? max(p, q) : min(p, q); };
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0xB1, 0xf, 0xf, false)));
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0x4E, 0xf, 0xf, false)));
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0x141, 0xf, 0xf, false)));
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0x140, 0xf, 0xf, false)));
  auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(p[0], p[1]);
  auto q = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(q[0], q[1]);
}

// hist: this wave's kWaveRadixPasses x 256 counters, all zero on entry.
template <int KR, typename TailKey>
__device__ __forceinline__ WaveSelection wave_select(const WaveKeys<KR>& wk, int nb, int topk, int (*hist)[256],
                                                     TailKey tail_key) {
  const int lane = threadIdx.x & 63;
  WaveSelection w;
  w.kk = min(topk, nb);
  w.partial = w.kk < nb;
  w.T = 0;
  w.need = 0;
  w.all_eq_kept = true;
  if (!w.partial) return w;
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < KR; ++i)
    if (lane + 64 * i < nb) {
      kmax = max(kmax, wk.k[i]);
      kmin = min(kmin, wk.k[i]);
    }
  for (int e = lane + 64 * KR; e < nb; e += 64) {
    const uint32_t k = tail_key(e);
    kmax = max(kmax, k);
    kmin = min(kmin, k);
  }
  // uniform after the reductions
  kmax = __builtin_amdgcn_readfirstlane(wave_extreme_u32<true>(kmax));
  kmin = __builtin_amdgcn_readfirstlane(wave_extreme_u32<false>(kmin));
  const uint32_t diff = kmax ^ kmin;
  if (diff == 0u) {  // every key is equal: the lowest K' ids
    w.T = kmax;
    w.need = w.kk;
    w.all_eq_kept = false;
    return w;
  }
  int top = 31 - __clz(diff);                                       // highest bit still open
  uint32_t prefix = (top == 31) ? 0u : (kmax & (~0u << (top + 1)));  // bits fixed so far
  int need = w.kk;
#pragma unroll 1
  for (int pass = 0; pass < kWaveRadixPasses; ++pass) {
    const int width = min(8, top + 1);
    const int shift = top + 1 - width;
    const uint32_t fixed = (top == 31) ? 0u : (~0u << (top + 1));
    const uint32_t dmask = (1u << width) - 1u;
    int* h = hist[pass];
    auto bin = [&](uint32_t k) {
      if ((k & fixed) == prefix) atomicAdd(&h[(k >> shift) & dmask], 1);
    };
#pragma unroll
    for (int i = 0; i < KR; ++i)
      if (lane + 64 * i < nb) bin(wk.k[i]);
    for (int e = lane + 64 * KR; e < nb; e += 64) bin(tail_key(e));
    wave_lds_order();
    // lane owns digits 255-4*lane .. 252-4*lane (descending)
    const i32x4 h4 = *reinterpret_cast<const i32x4*>(&h[252 - 4 * lane]);
    const int c[4] = {h4[3], h4[2], h4[1], h4[0]};
    const int local = c[0] + c[1] + c[2] + c[3];
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
    if (need == cnt) {
      // every key sharing the prefix so far is kept: keys >= prefix (lower
      // bits zero) are exactly the K' largest, no tie straddles the cut
      w.T = prefix;
      w.all_eq_kept = true;
      return w;
    }
    if (shift == 0) break;
    top = shift - 1;
  }
  w.T = prefix;
  w.need = need;
  w.all_eq_kept = false;  // keys equal to T straddle the cut: lowest ids first
  return w;
}

// Walks the kept blocks in ascending id order, 64 blocks at a time, keeping
// only population counts of the keep ballots, and calls found(rank, block,
// payload) for every rank in [q0, q1) (all arguments uniform, every lane
// calls it). payload is pay[i] of the lane holding the block in register
// slot i, or tail_pay(e) past the register slots. Returns the context
// length 128*K' - (block nb-1 kept ? 128*nb - v : 0) in every lane.
template <int KR, typename TailKey, typename TailPay, typename Found>
__device__ __forceinline__ int wave_locate(const WaveKeys<KR>& wk, const int (&pay)[KR], int nb, int v,
                                           const WaveSelection& w, int q0, int q1, TailKey tail_key,
                                           TailPay tail_pay, Found found) {
  const int lane = threadIdx.x & 63;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int carry = 0, carry_eq = 0, q = q0;
  bool last_kept = false;
  q1 = min(q1, w.kk);
  auto keep_of = [&](bool valid, uint32_t k) {
    if (!w.partial) return valid;
    if (w.all_eq_kept) return valid && k >= w.T;
    const bool eq = valid && k == w.T;
    const unsigned long long em = __ballot(eq);
    const int rank_eq = carry_eq + __popcll(em & lt);
    carry_eq += __popcll(em);
    return valid && (k > w.T || (eq && rank_eq < w.need));
  };
  // one chunk of 64 blocks starting at base; get_pay() gives the lane's payload
  auto chunk = [&](int base, uint32_t k, auto get_pay) {
    const bool keep = keep_of(base + lane < nb, k);
    const unsigned long long km = __ballot(keep);
    const int c = __popcll(km);
    if (nb - 1 - base < 64) last_kept = (km >> (nb - 1 - base)) & 1ull;
    if (q < q1 && q < carry + c) {
      const int below = __popcll(km & lt);
      const int p = get_pay();
      do {
        const unsigned long long hit = __ballot(keep && below == q - carry);
        const int src = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<unsigned long long>(hit)) - 1);
        found(q, base + src, __builtin_amdgcn_readlane(p, src));
        ++q;
      } while (q < q1 && q < carry + c);
    }
    carry += c;
  };
#pragma unroll
  for (int i = 0; i < KR; ++i)
    if (64 * i < nb) chunk(64 * i, wk.k[i], [&] { return pay[i]; });
  for (int base = 64 * KR; base < nb; base += 64) {
    const int e = min(base + lane, nb - 1);
    chunk(base, tail_key(e), [&] { return tail_pay(e); });
  }
  return kPage * w.kk - (last_kept ? kPage * nb - v : 0);
}

// ---------------------------------------------------------------------------
// The same selection with the four waves of a workgroup sharing the work:
// thread t holds the keys of blocks t + 256*i, i < KC (a row of at most
// 256*KC blocks), the radix histogram is shared, and every wave reads the
// same histogram after one barrier per pass, so all waves reach the same
// threshold. The keep ballots of 64-block chunks (chunk c = 4*i + wave) go to
// LDS, and each wave then looks up the ranks it needs.
// ---------------------------------------------------------------------------
constexpr int kCoopMaxChunks = 16;  // 1024 blocks

struct CoopLds {
  int hist[kWaveRadixPasses][256];  // cleared before the selection
  uint32_t ext[4][2];               // per-wave max / min key
  int eqc[kCoopMaxChunks];          // keys equal to the threshold, per chunk
  int cnt[kCoopMaxChunks];          // kept blocks per chunk
  unsigned long long mask[kCoopMaxChunks];
  int page[kCoopMaxChunks * 64];    // block-table entry of every kept block
};

// Clears the histograms (all 256 threads; the first barrier of coop_select
// orders it before any use).
__device__ __forceinline__ void coop_clear(CoopLds& L) {
  i32x4* h = reinterpret_cast<i32x4*>(&L.hist[0][0]);
  h[threadIdx.x] = i32x4{0, 0, 0, 0};
}

// Every thread of the workgroup calls it; the result is uniform.
template <int KC>
__device__ __forceinline__ WaveSelection coop_select(const uint32_t (&k)[KC], int nb, int topk, CoopLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  WaveSelection w;
  w.kk = min(topk, nb);
  w.partial = w.kk < nb;
  w.T = 0;
  w.need = 0;
  w.all_eq_kept = true;
  if (!w.partial) return w;
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < KC; ++i)
    if (tid + 256 * i < nb) {
      kmax = max(kmax, k[i]);
      kmin = min(kmin, k[i]);
    }
  kmax = wave_extreme_u32<true>(kmax);
  kmin = wave_extreme_u32<false>(kmin);
  if (lane == 0) {
    L.ext[wave][0] = kmax;
    L.ext[wave][1] = kmin;
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    kmax = max(kmax, L.ext[x][0]);
    kmin = min(kmin, L.ext[x][1]);
  }
  kmax = __builtin_amdgcn_readfirstlane(kmax);
  kmin = __builtin_amdgcn_readfirstlane(kmin);
  const uint32_t diff = kmax ^ kmin;
  if (diff == 0u) {  // every key is equal: the lowest K' ids
    w.T = kmax;
    w.need = w.kk;
    w.all_eq_kept = false;
    return w;
  }
  int top = 31 - __clz(diff);
  uint32_t prefix = (top == 31) ? 0u : (kmax & (~0u << (top + 1)));
  int need = w.kk;
#pragma unroll 1
  for (int pass = 0; pass < kWaveRadixPasses; ++pass) {
    const int width = min(8, top + 1);
    const int shift = top + 1 - width;
    const uint32_t fixed = (top == 31) ? 0u : (~0u << (top + 1));
    const uint32_t dmask = (1u << width) - 1u;
    int* h = L.hist[pass];
#pragma unroll
    for (int i = 0; i < KC; ++i)
      if (tid + 256 * i < nb && (k[i] & fixed) == prefix) atomicAdd(&h[(k[i] >> shift) & dmask], 1);
    __syncthreads();
    // lane owns digits 255-4*lane .. 252-4*lane (descending); every wave
    // scans the same counts
    const i32x4 h4 = *reinterpret_cast<const i32x4*>(&h[252 - 4 * lane]);
    const int c[4] = {h4[3], h4[2], h4[1], h4[0]};
    const int local = c[0] + c[1] + c[2] + c[3];
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
    const int src = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<unsigned long long>(__ballot(found))) - 1);
    prefix |= static_cast<uint32_t>(__builtin_amdgcn_readlane(my_digit, src)) << shift;
    need = __builtin_amdgcn_readlane(my_need, src);
    const int cnt = __builtin_amdgcn_readlane(my_cnt, src);
    if (need == cnt) {
      w.T = prefix;
      w.all_eq_kept = true;
      return w;
    }
    if (shift == 0) break;
    top = shift - 1;
  }
  w.T = prefix;
  w.need = need;
  w.all_eq_kept = false;
  return w;
}

// Keep ballots to LDS, then found(rank, block, page) for the ranks
// [q0, q1) this wave needs (uniform arguments). Every thread calls it.
// Returns the context length 128*K' - (block nb-1 kept ? 128*nb - v : 0).
template <int KC, typename Found>
__device__ __forceinline__ int coop_locate(const uint32_t (&k)[KC], const int (&pg)[KC], int nb, int v,
                                           const WaveSelection& w, int q0, int q1, CoopLds& L, Found found) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long lt = (1ull << lane) - 1ull;
  bool keep[KC];
  if (!w.partial || w.all_eq_kept) {
#pragma unroll
    for (int i = 0; i < KC; ++i) keep[i] = tid + 256 * i < nb && (!w.partial || k[i] >= w.T);
  } else {
    // ties straddle the cut: equal keys are kept in ascending block order
    unsigned long long em[KC];
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      em[i] = __ballot(tid + 256 * i < nb && k[i] == w.T);
      if (lane == 0) L.eqc[4 * i + wave] = __popcll(em[i]);
    }
    __syncthreads();
    const int ev = lane < 4 * KC ? L.eqc[lane] : 0;
    const int eincl = wave_inclusive_scan(ev);
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int before = __builtin_amdgcn_readlane(eincl - ev, 4 * i + wave);
      const bool eq = (em[i] >> lane) & 1ull;
      keep[i] = tid + 256 * i < nb && (k[i] > w.T || (eq && before + __popcll(em[i] & lt) < w.need));
    }
  }
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const unsigned long long km = __ballot(keep[i]);
    if (lane == 0) {
      L.mask[4 * i + wave] = km;
      L.cnt[4 * i + wave] = __popcll(km);
    }
    if (keep[i]) L.page[tid + 256 * i] = pg[i];
  }
  __syncthreads();
  const int nchunks = (nb + 63) >> 6;
  const int cv = lane < nchunks ? L.cnt[lane] : 0;
  const int cincl = wave_inclusive_scan(cv);
  q1 = min(q1, w.kk);
  for (int q = q0; q < q1; ++q) {
    const int c = __popcll(__ballot(lane < nchunks && cincl <= q));
    const int excl = __builtin_amdgcn_readlane(cincl - cv, c);
    const unsigned long long m = L.mask[c];
    const unsigned long long hit = __ballot(((m >> lane) & 1ull) && __popcll(m & lt) == q - excl);
    const int e = 64 * c + __builtin_amdgcn_readfirstlane(__ffsll(static_cast<unsigned long long>(hit)) - 1);
    found(q, e, L.page[e]);
  }
  const bool last_kept = nb > 0 && ((L.mask[(nb - 1) >> 6] >> ((nb - 1) & 63)) & 1ull);
  return kPage * w.kk - (last_kept ? kPage * nb - v : 0);
}

}  // namespace msa

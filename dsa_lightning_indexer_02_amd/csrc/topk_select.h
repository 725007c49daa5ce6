// Block-wide top-k selection over keys held in registers (shared by the top-k kernels and the fused
// indexer -> top-k): see topk.hip for the method.
#pragma once

#include "common.h"

namespace dsa {

constexpr int kTopkBlock = 1024;
constexpr int kTopkWaves = kTopkBlock / kWave;
constexpr int kBinBits = 11;
constexpr int kBins = 1 << kBinBits;

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int BLOCK>
struct TopkSharedT {
  uint32_t hist[kBins];
  uint32_t cnt[BLOCK];            // per-(item, wave) counts, then their exclusive scan
  uint32_t wave_tot[BLOCK / kWave];
  uint32_t red[2 * (BLOCK / kWave)];
  uint32_t bcast[4];
};
using TopkShared = TopkSharedT<kTopkBlock>;

// Inclusive prefix sum of one value per thread over the block, in thread order.
template <int BLOCK>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, TopkSharedT<BLOCK> &sh) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_incl_sum(v);
  if (lane == kWave - 1) sh.wave_tot[w] = v;
  __syncthreads();
  uint32_t add = 0;
  for (int i = 0; i < w; ++i) add += sh.wave_tot[i];
  __syncthreads();
  return v + add;
}

// Exclusive scan, in place, of sh.cnt[0 .. n_entries) (n_entries <= block size).
template <int BLOCK>
__device__ __forceinline__ void scan_counts(int n_entries, TopkSharedT<BLOCK> &sh) {
  const int t = threadIdx.x;
  const uint32_t v = t < n_entries ? sh.cnt[t] : 0u;
  const uint32_t inc = block_incl_scan(v, sh);
  if (t < n_entries) sh.cnt[t] = inc - v;
  __syncthreads();
}

// Select the top `k` of the `n` valid keys (item i of thread t is element L = i * BLOCK + t; elements
// with L >= n are absent) and call emit(rank, L, key) for each kept element, rank = its ascending-L slot.
template <int ITEMS, int BLOCK = kTopkBlock, class Emit>
__device__ __forceinline__ void select_topk(const uint32_t (&key)[ITEMS], int n, int k, Emit emit,
                                            TopkSharedT<BLOCK> &sh) {
  constexpr int WAVES = BLOCK / kWave;
  constexpr int BPT = kBins / BLOCK;   // bins owned by each thread in the bin scan
  static_assert(BLOCK % kWave == 0 && kBins % BLOCK == 0 && ITEMS * WAVES <= BLOCK, "select tiling");
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  if (n <= k) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int L = i * BLOCK + tid;
      if (L < n && L < k) emit(L, L, key[i]);
    }
    return;
  }
  // --- key range of the row
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    if (i * BLOCK + tid < n) {
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
  }
  kmin = wave_total_min(kmin);
  kmax = wave_total_max(kmax);
  if (lane == 0) {
    sh.red[w] = kmin;
    sh.red[WAVES + w] = kmax;
  }
  __syncthreads();
  kmin = sh.red[0];
  kmax = sh.red[WAVES];
  for (int i = 1; i < WAVES; ++i) {
    kmin = min(kmin, sh.red[i]);
    kmax = max(kmax, sh.red[WAVES + i]);
  }
  // --- bucket passes: the window [lo, hi] holds the k-th best key and `need` of the keys inside it are
  //     still to be taken; each pass splits the window into at most 2048 bins of width 2^shift.
  uint32_t lo = kmin, hi = kmax;
  const uint32_t range = kmax - kmin;
  int shift = range == 0u ? 0 : max(0, 32 - __clz((int)range) - kBinBits);
  uint32_t need = (uint32_t)k;
  uint32_t T, cnt_eq;
  while (true) {
    for (int b = tid; b < kBins; b += BLOCK) sh.hist[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      if (i * BLOCK + tid < n && key[i] >= lo && key[i] <= hi) atomicAdd(&sh.hist[(key[i] - lo) >> shift], 1u);
    }
    __syncthreads();
    // thread t owns BPT consecutive bins counted from the top: kBins-1-BPT*t down to kBins-BPT*(t+1)
    const int hb = kBins - 1 - BPT * tid;
    uint32_t cb[BPT], csum = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      cb[j] = sh.hist[hb - j];
      csum += cb[j];
    }
    const uint32_t incl = block_incl_scan(csum, sh);   // keys in bins >= hb - BPT + 1
    uint32_t run = incl - csum;                        // keys in bins > hb
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      if (run < need && need <= run + cb[j]) {
        sh.bcast[0] = (uint32_t)(hb - j); sh.bcast[1] = run; sh.bcast[2] = cb[j];
      }
      run += cb[j];
    }
    __syncthreads();
    const uint32_t B = sh.bcast[0], above = sh.bcast[1], inbin = sh.bcast[2];
    need -= above;
    lo += B << shift;
    hi = (uint32_t)min((uint64_t)hi, (uint64_t)lo + ((1ull << shift) - 1ull));
    if (shift == 0) {
      T = lo;
      cnt_eq = inbin;
      break;
    }
    shift = max(0, shift - kBinBits);
    __syncthreads();  // everyone has read bcast before the next pass rewrites it
  }
  // --- ordered compaction
  const bool take_all_eq = (need == cnt_eq);
  const int n_entries = ITEMS * WAVES;
  if (!take_all_eq) {
    // position-order rank of each T-valued key: only the first `need` of them are kept
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const bool eq = (i * BLOCK + tid < n) && key[i] == T;
      const uint64_t m = ballot(eq);
      if (lane == 0) sh.cnt[i * WAVES + w] = (uint32_t)__popcll(m);
    }
    __syncthreads();
    scan_counts(n_entries, sh);
  }
  uint64_t selbits = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const bool valid = i * BLOCK + tid < n;
    bool s = valid && key[i] > T;
    const bool eq = valid && key[i] == T;
    if (take_all_eq) {
      s = s || eq;
    } else {
      // entry (i, w) belongs to this wave alone: its tie base is read before lane 0 reuses it below
      const uint64_t m = ballot(eq);
      const uint32_t r = sh.cnt[i * WAVES + w] + (uint32_t)lanes_below(m);
      s = s || (eq && r < need);
    }
    selbits |= (uint64_t)s << i;
    const uint64_t m = ballot(s);
    if (lane == 0) sh.cnt[i * WAVES + w] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  scan_counts(n_entries, sh);
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const bool s = (selbits >> i) & 1u;
    const uint64_t m = ballot(s);
    if (s) {
      const int rank = (int)sh.cnt[i * WAVES + w] + lanes_below(m);
      if (rank < k) emit(rank, i * BLOCK + tid, key[i]);  // exactly k are selected; the guard only bounds writes
    }
  }
}


}  // namespace dsa

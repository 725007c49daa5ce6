// Causal top-k selection for DSA: per query row, keep the k best-scoring positions among 0..p.
//
// Defined by the GLM sparse-attention essay (needle paragraph: the cut-off is the k-th best score) and
// "Sparse Attention Architecture Evolution in LLMs", section "Top-K Selection: A Hard Filtering Mechanism"
// (a hard budget of k positions per query token). Ties go to the lower position and -0.0 ranks as +0.0;
// the kept positions are written in ascending order, padded with -1.
//
// Method (one workgroup of 1024 threads per row, the row held in registers):
//   1. scores -> order-preserving uint32 keys (larger score <=> larger key);
//   2. bucket select in LDS: bins are the row's own key range [min, max] split into 2048 equal bins, so the
//      bins adapt to however narrow the score distribution is; the bin holding the k-th best key is
//      refined the same way (at most three passes for 32-bit keys) until the exact threshold key T and the
//      number of T-valued keys still to take are known;
//   3. ordered compaction: wave ballots give per-(item, wave) counts, one block scan of those counts gives
//      every selected element its output slot in position order, so the output is ascending with no sort.
// Batches with too few rows to fill the GPU (decode) split each row into chunks that keep only the keys of a
// sampled window (windowed form below), and a second pass selects k among those candidates.
#include "common.h"
#include "kernels.h"
#include "topk_select.h"

namespace dsa {

// One workgroup per query row; the whole row (<= ITEMS * 1024 scores) in registers.
template <int ITEMS>
__global__ __launch_bounds__(kTopkBlock) void topk_rows_kernel(const float *__restrict__ scores, int64_t ld,
                                                              const int32_t *__restrict__ q_pos, int k,
                                                              int32_t *__restrict__ idx) {
  __shared__ TopkShared sh;
  const int r = blockIdx.x;
  const int n = q_pos[r] + 1;
  int32_t *out = idx + (int64_t)r * k;
  if (n <= k) {
    for (int j = threadIdx.x; j < k; j += kTopkBlock) out[j] = j < n ? j : -1;
    return;
  }
  const float *row = scores + (int64_t)r * ld;
  // every item loads (past the row's end the row's last score, replaced below) so that no branch separates
  // the loads: they go out together and the row pays one memory latency
  float v[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) v[i] = row[min(i * kTopkBlock + (int)threadIdx.x, n - 1)];
  uint32_t key[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) key[i] = i * kTopkBlock + (int)threadIdx.x < n ? order_key(v[i]) : 0u;
  select_topk<ITEMS>(key, n, k, [&](int rank, int L, uint32_t) { out[rank] = L; }, sh);
}

// Merge of the fused indexer -> top-k: select k among the row's candidates, chunk c's own top-k at slot
// (r * n_chunks + c) * k. Chunks before the last one each hold exactly k candidates (chunk >= k), so the
// candidates of a row are contiguous and in position order.
template <int ITEMS>
__global__ __launch_bounds__(kTopkBlock) void topk_merge_kernel(const int32_t *__restrict__ q_pos, int k,
                                                               int chunk, int n_chunks,
                                                               const uint32_t *__restrict__ cand_key,
                                                               const int32_t *__restrict__ cand_pos,
                                                               int32_t *__restrict__ idx) {
  __shared__ TopkShared sh;
  const int r = blockIdx.x;
  const int n = q_pos[r] + 1;
  int32_t *out = idx + (int64_t)r * k;
  if (n <= k) {
    for (int j = threadIdx.x; j < k; j += kTopkBlock) out[j] = j < n ? j : -1;
    return;
  }
  const int used = (n + chunk - 1) / chunk;
  const int last_len = n - (used - 1) * chunk;
  const int total = (used - 1) * k + min(last_len, k);
  const int64_t base = (int64_t)r * n_chunks * k;
  // Up to 32 items a thread, keys and positions load together and branch-free, as in the rows form (past the
  // last candidate the last one is loaded, then replaced), and the output pass only stores (item i is
  // L = i * kTopkBlock + tid). At 64 the positions would not fit in registers beside the keys (and the clamped
  // addresses spill): the keys load masked and the positions are read per output.
  constexpr bool kPosInRegs = ITEMS <= 32;
  uint32_t key[ITEMS];
  int32_t pos[kPosInRegs ? ITEMS : 1];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int L = i * kTopkBlock + (int)threadIdx.x;
    if constexpr (kPosInRegs) {
      const int64_t c = base + min(L, total - 1);
      key[i] = cand_key[c];
      pos[i] = cand_pos[c];
    } else {
      key[i] = L < total ? cand_key[base + L] : 0u;
    }
  }
  if constexpr (kPosInRegs) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) key[i] = i * kTopkBlock + (int)threadIdx.x < total ? key[i] : 0u;
  }
  select_topk<ITEMS>(
      key, total, k,
      [&](int rank, int L, uint32_t) {
        if constexpr (kPosInRegs)
          out[rank] = pos[(L - (int)threadIdx.x) / kTopkBlock];
        else
          out[rank] = cand_pos[base + L];
      },
      sh);
}

// ---------------------------------------------------------------------------------------------------------
// Streaming form for long rows (one 256-thread workgroup per row, nothing held in registers across passes).
// Wave w owns the contiguous segment [w*seg, (w+1)*seg) of the row, so walking the segments in wave order
// visits positions in ascending order and each wave's output base is a prefix sum of per-wave counts.
//   1. a sample of 4096 keys (64 stratified runs of 64 consecutive keys, so the sample reads 16 KB, not the
//      row), histogrammed over its own range, brackets the k-th key in a window [lo, hi] with a statistical
//      margin (3 standard deviations of the sample count, plus 2);
//   2. one pass over the row keeps every key >= lo, with its position, in the wave's LDS region (in position
//      order), and counts the keys above the window (16-byte loads, 4 positions per lane, when the rows are
//      16-byte aligned);
//   3. a bucket search over the window's keys (each lane's share of its wave's LDS region loaded into registers
//      once) finds the exact threshold T and how many T-valued keys are taken (lowest positions first); each
//      wave then writes its kept positions, in order.
// The row is read from HBM once. When the window misses the k-th key, or a wave's keys overflow its region,
// a streaming bucket select over the whole row finds T instead (three passes of 11, 11 and 10 key bits),
// followed by a counting pass and an output pass.
constexpr int kStreamWaves = 4;
constexpr int kStreamThreads = kStreamWaves * kWave;
constexpr int kStreamUnroll = 16;          // loads in flight per wave
constexpr int kRun = kWave;                // sample runs of 64 consecutive keys
constexpr int kRuns = 64;
constexpr int kSample = kRuns * kRun;      // 4096 sampled keys per row
constexpr int kCandPerWave = 1016;         // candidate (key, position) pairs one wave keeps: 4 workgroups per CU

// Shared state of a W-wave workgroup: the same candidate capacity in all (W regions of CPW pairs).
template <int W>
struct StreamSharedT {
  static constexpr int CPW = kStreamWaves * kCandPerWave / W;   // candidate pairs per wave region
  uint32_t hist[kBins];
  uint32_t cand_key[W * CPW];
  int32_t cand_pos[W * CPW];
  uint32_t wave_tot[W];
  uint32_t red[4 * W];
  uint32_t bcast[6];
};
using StreamShared = StreamSharedT<kStreamWaves>;

// Inclusive prefix sum over the block, in thread order.
template <int W>
__device__ __forceinline__ uint32_t stream_incl_scan(uint32_t v, StreamSharedT<W> &sh) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_incl_sum(v);
  if (lane == kWave - 1) sh.wave_tot[w] = v;
  __syncthreads();
  uint32_t add = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) add += i < w ? sh.wave_tot[i] : 0u;
  __syncthreads();
  return v + add;
}

// Bins counted from the top (bin kBins-1 first). For each rank r[q] (1-based, 1 <= r[q] <= total), writes
// to sh.bcast[3q..3q+2] the bin holding the r[q]-th key, the number of keys in higher bins, and its count.
template <int NR, int W>
__device__ __forceinline__ void stream_rank_bins(StreamSharedT<W> &sh, const int (&r)[NR]) {
  constexpr int BPT = kBins / (W * kWave);              // bins per thread
  const int tid = threadIdx.x;
  const int top = kBins - 1 - BPT * tid;                // this thread's bins: top, top-1, .., top-BPT+1
  uint32_t c[BPT], sum = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    c[j] = sh.hist[top - j];
    sum += c[j];
  }
  const uint32_t incl = stream_incl_scan(sum, sh);
  uint32_t above = incl - sum;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      if (above < (uint32_t)r[q] && (uint32_t)r[q] <= above + c[j]) {
        sh.bcast[3 * q] = (uint32_t)(top - j);
        sh.bcast[3 * q + 1] = above;
        sh.bcast[3 * q + 2] = c[j];
      }
    }
    above += c[j];
  }
  __syncthreads();
}

template <int W>
__device__ __forceinline__ void stream_clear_hist(StreamSharedT<W> &sh) {
  for (int b = threadIdx.x; b < kBins; b += W * kWave) sh.hist[b] = 0u;
}

// The k-th largest key of the whole row by streaming bucket passes over the row (exact; used when the sampled
// window misses). Bins cover the key bits 31..21, then 20..10, then 9..0 of the window.
template <int W>
__device__ __forceinline__ void stream_threshold(const float *__restrict__ row, int n, int k, StreamSharedT<W> &sh,
                                                 uint32_t &T, uint32_t &need_eq, uint32_t &cnt_eq) {
  const int tid = threadIdx.x;
  uint32_t lo = 0u, hi = 0xffffffffu, need = (uint32_t)k;
  int shift = 32 - kBinBits;
  while (true) {
    __syncthreads();
    stream_clear_hist(sh);
    __syncthreads();
    for (int L = tid; L < n; L += W * kWave) {
      const uint32_t x = order_key(row[L]);
      if (x >= lo && x <= hi) atomicAdd(&sh.hist[(x - lo) >> shift], 1u);
    }
    __syncthreads();
    const int rr[1] = {(int)need};
    stream_rank_bins<1>(sh, rr);
    const uint32_t B = sh.bcast[0], above = sh.bcast[1], inbin = sh.bcast[2];
    need -= above;
    lo += B << shift;
    hi = (uint32_t)min((uint64_t)hi, (uint64_t)lo + ((1ull << shift) - 1ull));
    if (shift == 0) {
      T = lo;
      cnt_eq = inbin;
      need_eq = need;
      break;
    }
    shift = max(0, shift - kBinBits);
  }
  __syncthreads();
}

// Walks the wave's segment [s0, s1) in 64-element steps, kStreamUnroll loads in flight; f(L, key, valid) is
// called for each step in position order (L = this lane's position).
template <class F>
__device__ __forceinline__ void stream_segment(const float *__restrict__ row, int s0, int s1, F f) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int L0 = s0; L0 < s1; L0 += kWave * kStreamUnroll) {
    float v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int L = L0 + u * kWave + lane;
      v[u] = L < s1 ? row[L] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int L = L0 + u * kWave + lane;
      f(L, order_key(v[u]), L < s1);
    }
  }
}

// Exclusive prefix over the lanes of a per-lane count c in 0..7 (three ballots), and the wave's total.
__device__ __forceinline__ uint32_t lane_prefix8(uint32_t c, uint32_t &total) {
  const uint64_t b0 = ballot(c & 1u), b1 = ballot(c & 2u), b2 = ballot(c & 4u);
  total = (uint32_t)__popcll(b0) + 2u * (uint32_t)__popcll(b1) + 4u * (uint32_t)__popcll(b2);
  return (uint32_t)lanes_below(b0) + 2u * (uint32_t)lanes_below(b1) + 4u * (uint32_t)lanes_below(b2);
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) { return wave_total_sum(v); }

// ---- 1. sample: run b (0..63) starts at floor(b * (n - 64) / 63); wave w of W reads runs w*64/W .. (w+1)*64/W - 1.
//      Gives the window [lo, hi] (lo = 0 / hi = ~0 when the margin reaches past the sample). Uses hist, red, bcast.
template <int W>
__device__ __forceinline__ void stream_window(const float *__restrict__ row, int n, int k, StreamSharedT<W> &sh,
                                              uint32_t &lo, uint32_t &hi) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  constexpr int SP = kSample / (W * kWave);   // sample runs per wave
  uint32_t sk[SP];
#pragma unroll
  for (int j = 0; j < SP; ++j) {
    const int b = w * SP + j;
    const int start = (int)(((int64_t)b * max(0, n - kRun)) / (kRuns - 1));
    sk[j] = order_key(row[min(n - 1, start + lane)]);
  }
  uint32_t smin = sk[0], smax = sk[0];
#pragma unroll
  for (int j = 1; j < SP; ++j) {
    smin = min(smin, sk[j]);
    smax = max(smax, sk[j]);
  }
  smin = wave_total_min(smin);
  smax = wave_total_max(smax);
  stream_clear_hist(sh);
  if (lane == 0) {
    sh.red[w] = smin;
    sh.red[W + w] = smax;
  }
  __syncthreads();
  smin = sh.red[0];
  smax = sh.red[W];
#pragma unroll
  for (int i = 1; i < W; ++i) {
    smin = min(smin, sh.red[i]);
    smax = max(smax, sh.red[W + i]);
  }
  const uint32_t range = smax - smin;
  const int shift = range == 0u ? 0 : max(0, 32 - __clz((int)range) - kBinBits);
#pragma unroll
  for (int j = 0; j < SP; ++j) atomicAdd(&sh.hist[(sk[j] - smin) >> shift], 1u);
  // sample ranks (from the top) around the k-th key: expected E = kSample k / n, margin 3 sd + 2
  const float p = (float)k / (float)n;
  const float E = p * (float)kSample, M = 3.f * sqrtf(E * (1.f - p)) + 2.f;
  const int r_hi = (int)floorf(E - M);    // the window's top lies below the (r_hi + 1)-th sample
  const int r_lo = (int)ceilf(E + M);     // its bottom at or below the r_lo-th sample
  __syncthreads();
  {
    const int rr[2] = {max(1, min(kSample, r_hi + 1)), max(1, min(kSample, r_lo))};
    stream_rank_bins<2>(sh, rr);
  }
  hi = 0xffffffffu;
  lo = 0u;
  if (r_hi >= 0 && r_hi + 1 <= kSample)
    hi = (uint32_t)min((uint64_t)0xffffffffu, (uint64_t)smin + ((uint64_t)(sh.bcast[0] + 1) << shift) - 1ull);
  if (r_lo <= kSample) lo = smin + (sh.bcast[3] << shift);
}

// ---- 2. one pass over this wave's segment [s0, s1): every key >= lo with its position goes to the wave's LDS
//      region (position order; cc counts them all, only the first kCandPerWave are stored), and ca counts the
//      keys above hi.
// 16-byte form (rows 16-byte aligned): lane l takes positions L .. L+3, L = L0 + 4l (lane order is position
// order), kCollectU loads per lane a batch. Loads are clamped to the segment's last aligned position (nothing
// past the row is read; the positions past s1 are masked by their count), so a batch issues without a branch:
// the caller loads the first batch before the window is known, and each step issues the next batch before
// processing the current one, so the loads of a batch overlap the processing of the one before.
constexpr int kCollectU = 4;
__device__ __forceinline__ void stream_load4(const float *__restrict__ row, int L0, int s1, f32x4 (&v)[kCollectU]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int last = max(0, (s1 - 1) & ~3);
#pragma unroll
  for (int u = 0; u < kCollectU; ++u) v[u] = *(const f32x4 *)(row + min(L0 + u * 4 * kWave + 4 * lane, last));
}

__device__ __forceinline__ void stream_collect4(const float *__restrict__ row, int s0, int s1, uint32_t lo,
                                                uint32_t hi, StreamShared &sh, f32x4 (&a)[kCollectU], uint32_t &ca,
                                                uint32_t &cc) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int cb = w * kCandPerWave;
  constexpr int STEP = 4 * kWave * kCollectU;
  uint32_t ca_lane = 0u, ccl = 0u;
  auto process = [&](int L0, const f32x4 (&v)[kCollectU]) {
#pragma unroll
    for (int u = 0; u < kCollectU; ++u) {
      const int L = L0 + u * 4 * kWave + 4 * lane;
      const int nv = min(4, max(0, s1 - L));
      const uint32_t x[4] = {order_key(v[u].x), order_key(v[u].y), order_key(v[u].z), order_key(v[u].w)};
      uint32_t nc = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ca_lane += (j < nv && x[j] > hi) ? 1u : 0u;
        nc += (j < nv && x[j] >= lo) ? 1u : 0u;
      }
      uint32_t tot;
      uint32_t slot = ccl + lane_prefix8(nc, tot);
      if (tot != 0u) {   // wave-uniform
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j < nv && x[j] >= lo) {
            if (slot < (uint32_t)kCandPerWave) {
              sh.cand_key[cb + slot] = x[j];
              sh.cand_pos[cb + slot] = L + j;
            }
            ++slot;
          }
        }
      }
      ccl += tot;
    }
  };
  f32x4 b[kCollectU];
  for (int L0 = s0; L0 < s1;) {   // two batches a trip, so the buffers swap roles without register copies
    stream_load4(row, L0 + STEP, s1, b);
    process(L0, a);
    L0 += STEP;
    if (L0 >= s1) break;
    stream_load4(row, L0 + STEP, s1, a);
    process(L0, b);
    L0 += STEP;
  }
  ca = wave_sum_u32(ca_lane);
  cc = ccl;
}

// Element-wise form (any alignment).
__device__ __forceinline__ void stream_collect(const float *__restrict__ row, int s0, int s1, uint32_t lo,
                                               uint32_t hi, StreamShared &sh, uint32_t &ca, uint32_t &cc) {
  const int w = threadIdx.x / kWave;
  const int cb = w * kCandPerWave;
  uint32_t cal = 0u, ccl = 0u;
  stream_segment(row, s0, s1, [&](int L, uint32_t x, bool valid) {
    cal += (uint32_t)__popcll(ballot(valid && x > hi));
    const bool c = valid && x >= lo;
    const uint64_t bm = ballot(c);
    const uint32_t slot = ccl + (uint32_t)lanes_below(bm);
    if (c && slot < (uint32_t)kCandPerWave) {
      sh.cand_key[cb + slot] = x;
      sh.cand_pos[cb + slot] = L;
    }
    ccl += (uint32_t)__popcll(bm);
  });
  ca = cal;
  cc = ccl;
}

// Output slots of the kept keys: keys > T, and the first need_eq T-valued keys in position order (wave order,
// then in order within a wave). gt_w / eq_w: this wave's counts. Gives the wave's first slot and how many of its
// T-valued keys it takes. Starts with a barrier (red is reused).
template <int W>
__device__ __forceinline__ void stream_out_base(uint32_t gt_w, uint32_t eq_w, uint32_t need_eq, StreamSharedT<W> &sh,
                                                uint32_t &base, uint32_t &quota) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) {
    sh.red[w] = gt_w;
    sh.red[W + w] = eq_w;
  }
  __syncthreads();
  uint32_t eq_before = 0u;
  base = 0u;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    if (i < w) {
      const uint32_t ei = sh.red[W + i];
      const uint32_t take_i = min(ei, need_eq > eq_before ? need_eq - eq_before : 0u);
      base += sh.red[i] + take_i;
      eq_before += ei;
    }
  }
  quota = min(eq_w, need_eq > eq_before ? need_eq - eq_before : 0u);
}

// The ordered output walk: put(L, key, valid) is called in position order for this wave's elements;
// emit(slot, L, key) for every kept one (slot < limit).
template <class Emit>
struct StreamPut {
  uint32_t T, quota, base, eq_run, limit;
  Emit emit;
  __device__ __forceinline__ void operator()(int L, uint32_t x, bool valid) {
    const bool eq = valid && x == T;
    const uint64_t em = ballot(eq);
    const bool take = (valid && x > T) || (eq && eq_run + (uint32_t)lanes_below(em) < quota);
    eq_run += (uint32_t)__popcll(em);
    const uint64_t sm = ballot(take);
    if (take) {
      const uint32_t slot = base + (uint32_t)lanes_below(sm);
      if (slot < limit) emit(slot, L, x);   // exactly `limit` are taken; the guard only bounds the writes
    }
    base += (uint32_t)__popcll(sm);
  }
};

// Emit the kept keys of this wave's row segment [s0, s1), read again from the scores.
template <class Emit, int W>
__device__ __forceinline__ void stream_emit_row(const float *__restrict__ row, int s0, int s1, uint32_t T,
                                                uint32_t need_eq, uint32_t limit, StreamSharedT<W> &sh, Emit emit) {
  uint32_t g = 0u, e = 0u;
  stream_segment(row, s0, s1, [&](int, uint32_t x, bool valid) {
    g += (uint32_t)__popcll(ballot(valid && x > T));
    e += (uint32_t)__popcll(ballot(valid && x == T));
  });
  uint32_t base, quota;
  stream_out_base(g, e, need_eq, sh, base, quota);
  StreamPut<Emit> put{T, quota, base, 0u, limit, emit};
  stream_segment(row, s0, s1, [&](int L, uint32_t x, bool valid) { put(L, x, valid); });
}

// Selection among the candidates of the four wave LDS regions (wave v's region holds ccs[v] <= kCandPerWave
// (key, position) pairs in position order): the `need` largest of the keys <= top are kept, together with every
// candidate above top; emit(slot, position, key) for each kept one (slot < limit), in position order (wave order,
// then region order). Each lane loads its region entries j = u * 64 + lane into registers once, so the bucket
// passes count from registers, with no LDS reads between them. The passes stop as soon as the bin holding the
// need-th key is to be kept whole: then every key >= the bin's lower bound is kept (T = that bound, all T-valued).
constexpr int kRegItems = (kCandPerWave + kWave - 1) / kWave;   // 16
template <class Emit>
__device__ __forceinline__ void regions_select_emit(const uint32_t (&ccs)[kStreamWaves], uint32_t top, uint32_t need,
                                                    uint32_t limit, StreamShared &sh, Emit emit) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int cb = w * kCandPerWave;
  const uint32_t cnt = ccs[w];
  uint32_t key[kRegItems];
  int32_t pos[kRegItems];
#pragma unroll
  for (int u = 0; u < kRegItems; ++u) {
    const uint32_t j = (uint32_t)(u * kWave + lane);
    key[u] = j < cnt ? sh.cand_key[cb + j] : 0u;
    pos[u] = j < cnt ? sh.cand_pos[cb + j] : 0;
  }
  auto in_win = [&](int u) { return (uint32_t)(u * kWave + lane) < cnt && key[u] <= top; };
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int u = 0; u < kRegItems; ++u) {
    if (in_win(u)) {
      kmin = min(kmin, key[u]);
      kmax = max(kmax, key[u]);
    }
  }
  kmin = wave_total_min(kmin);
  kmax = wave_total_max(kmax);
  __syncthreads();   // red and bcast are free
  if (lane == 0) {
    sh.red[w] = kmin;
    sh.red[kStreamWaves + w] = kmax;
  }
  __syncthreads();
  kmin = sh.red[0];
  kmax = sh.red[kStreamWaves];
#pragma unroll
  for (int i = 1; i < kStreamWaves; ++i) {
    kmin = min(kmin, sh.red[i]);
    kmax = max(kmax, sh.red[kStreamWaves + i]);
  }
  uint32_t lo = kmin, hi = kmax, T, need_eq;
  const uint32_t range = kmax - kmin;
  int shift = range == 0u ? 0 : max(0, 32 - __clz((int)range) - kBinBits);
  while (true) {
    __syncthreads();
    stream_clear_hist(sh);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kRegItems; ++u)
      if (in_win(u) && key[u] >= lo && key[u] <= hi) atomicAdd(&sh.hist[(key[u] - lo) >> shift], 1u);
    __syncthreads();
    const int rr[1] = {(int)need};
    stream_rank_bins<1>(sh, rr);
    const uint32_t B = sh.bcast[0], above = sh.bcast[1], inbin = sh.bcast[2];
    need -= above;
    lo += B << shift;
    hi = (uint32_t)min((uint64_t)hi, (uint64_t)lo + ((1ull << shift) - 1ull));
    if (shift == 0 || inbin == need) {   // every key of the bin is kept: it is enough to keep all keys >= lo
      T = lo;
      need_eq = shift == 0 ? need : 0xffffffffu;
      break;
    }
    shift = max(0, shift - kBinBits);
  }
  uint32_t g = 0u, e = 0u;
#pragma unroll
  for (int u = 0; u < kRegItems; ++u) {
    const bool in = (uint32_t)(u * kWave + lane) < cnt;
    g += (uint32_t)__popcll(ballot(in && key[u] > T));
    e += (uint32_t)__popcll(ballot(in && key[u] == T));
  }
  uint32_t base, quota;
  stream_out_base(g, e, need_eq, sh, base, quota);
  StreamPut<Emit> put{T, quota, base, 0u, limit, emit};
#pragma unroll
  for (int u = 0; u < kRegItems; ++u) {
    const bool in = (uint32_t)(u * kWave + lane) < cnt;
    put(pos[u], key[u], in);
  }
}

// Selection of the k best among the windowed form's candidates (W wave LDS regions, as above), given the
// row's window [lo, top]. Only candidates >= lo count: when they number k or more the row's k-th key is >= lo,
// and then every position of the row's top-k is a candidate (a chunk keeps all its keys >= lo, or its own exact
// top-cap when it has more than cap of them). One histogram pass over [lo, top] (kBins bins) finds the bin of
// the k-th key; the few candidates in that bin are ranked against each other to give the exact threshold T and
// the number of T-valued keys to take. Returns false, having emitted nothing, when the window does not settle
// it: fewer than k candidates >= lo, k or more above top, or more than W * 64 candidates in the bin;
// the caller then selects over the whole row.
template <class Emit, int W>
__device__ __forceinline__ bool window_select_emit(const uint32_t (&ccs)[W], uint32_t lo, uint32_t top,
                                                   uint32_t k, StreamSharedT<W> &sh, Emit emit) {
  constexpr int CPW = StreamSharedT<W>::CPW, ITEMS = (CPW + kWave - 1) / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int cb = w * CPW;
  const uint32_t cnt = ccs[w];
  uint32_t key[ITEMS];
  int32_t pos[ITEMS];
#pragma unroll
  for (int u = 0; u < ITEMS; ++u) {
    const uint32_t j = (uint32_t)(u * kWave + lane);
    key[u] = j < cnt ? sh.cand_key[cb + j] : 0u;
    pos[u] = j < cnt ? sh.cand_pos[cb + j] : 0;
  }
  const uint32_t range = top - lo;   // top >= lo (both come from the same sample)
  const int shift = range == 0u ? 0 : max(0, 32 - __clz((int)range) - kBinBits);
  __syncthreads();   // the regions are in registers; hist, red and bcast are free
  stream_clear_hist(sh);
  if (tid == 0) sh.bcast[5] = 0u;
  __syncthreads();
  uint32_t a = 0u, in = 0u;
#pragma unroll
  for (int u = 0; u < ITEMS; ++u) {
    const bool v = (uint32_t)(u * kWave + lane) < cnt;
    const bool above = v && key[u] > top, inw = v && key[u] >= lo && key[u] <= top;
    a += (uint32_t)__popcll(ballot(above));
    in += (uint32_t)__popcll(ballot(inw));
    if (inw) atomicAdd(&sh.hist[(key[u] - lo) >> shift], 1u);
  }
  if (lane == 0) {
    sh.red[w] = a;
    sh.red[W + w] = in;
  }
  __syncthreads();
  uint32_t above = 0u, inwin = 0u;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    above += sh.red[i];
    inwin += sh.red[W + i];
  }
  if (above >= k || above + inwin < k) return false;   // block-uniform
  const int rr[1] = {(int)(k - above)};
  stream_rank_bins<1>(sh, rr);   // ends with a barrier
  const uint32_t B = sh.bcast[0], cnt_b = sh.bcast[2];
  const uint32_t need_b = k - above - sh.bcast[1];   // 1 <= need_b <= cnt_b
  const uint32_t blo = lo + (B << shift);
  const uint32_t bhi = (uint32_t)min((uint64_t)top, (uint64_t)blo + ((1ull << shift) - 1ull));
  uint32_t T, need_eq;
  if (shift == 0 || cnt_b == need_b) {   // the bin is one key value, or it is kept whole
    T = blo;
    need_eq = shift == 0 ? need_b : 0xffffffffu;
  } else {
    if (cnt_b > (uint32_t)(W * kWave)) return false;   // block-uniform (read from bcast)
    // the bin's keys -> a list in hist (free after the rank step), in any order; each thread then ranks one
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      const bool v = (uint32_t)(u * kWave + lane) < cnt;
      if (v && key[u] >= blo && key[u] <= bhi) sh.hist[atomicAdd(&sh.bcast[5], 1u)] = key[u];
    }
    __syncthreads();
    if ((uint32_t)tid < cnt_b) {
      const uint32_t x = sh.hist[tid];
      uint32_t gt = 0u, eq = 0u;
      for (uint32_t j = 0; j < cnt_b; ++j) {
        const uint32_t y = sh.hist[j];
        gt += y > x ? 1u : 0u;
        eq += y == x ? 1u : 0u;
      }
      if (gt < need_b && need_b <= gt + eq) {   // x is the need_b-th largest of the bin (equal x agree)
        sh.bcast[3] = x;
        sh.bcast[4] = need_b - gt;
      }
    }
    __syncthreads();
    T = sh.bcast[3];
    need_eq = sh.bcast[4];
  }
  uint32_t g = 0u, e = 0u;
#pragma unroll
  for (int u = 0; u < ITEMS; ++u) {
    const bool v = (uint32_t)(u * kWave + lane) < cnt;
    g += (uint32_t)__popcll(ballot(v && key[u] > T));
    e += (uint32_t)__popcll(ballot(v && key[u] == T));
  }
  uint32_t base, quota;
  stream_out_base(g, e, need_eq, sh, base, quota);
  StreamPut<Emit> put{T, quota, base, 0u, k, emit};
#pragma unroll
  for (int u = 0; u < ITEMS; ++u) {
    const bool v = (uint32_t)(u * kWave + lane) < cnt;
    put(pos[u], key[u], v);
  }
  return true;
}

// Per-wave counts after stream_collect: the totals, and whether every wave's keys fit its region.
template <int W>
__device__ __forceinline__ void stream_counts(uint32_t ca, uint32_t cc, StreamSharedT<W> &sh, uint32_t (&ccs)[W],
                                              uint32_t &c_above, uint32_t &c_cand, bool &fits) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  __syncthreads();   // bcast and red are free again
  if (lane == 0) {
    sh.red[w] = ca;
    sh.red[W + w] = cc;
  }
  __syncthreads();
  c_above = 0u;
  c_cand = 0u;
  fits = true;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    ccs[i] = sh.red[W + i];
    c_above += sh.red[i];
    c_cand += ccs[i];
    fits = fits && ccs[i] <= (uint32_t)StreamSharedT<W>::CPW;
  }
}

// Segments of the W waves over [0, n): starts at multiples of 256 positions (16-byte aligned when the row is).
template <int W = kStreamWaves>
__device__ __forceinline__ void stream_segment_of(int n, int &s0, int &s1) {
  const int w = threadIdx.x / kWave;
  const int seg = ((n + W - 1) / W + 4 * kWave - 1) / (4 * kWave) * (4 * kWave);
  s0 = min(n, w * seg);
  s1 = min(n, s0 + seg);
}

__global__ __launch_bounds__(kStreamThreads) void topk_stream_kernel(const float *__restrict__ scores, int64_t ld,
                                                                     const int32_t *__restrict__ q_pos, int num_q,
                                                                     int k, int32_t *__restrict__ idx) {
  __shared__ StreamShared sh;
  const int r = num_q - 1 - (int)blockIdx.x;    // longest rows of a prefill first
  const int n = q_pos[r] + 1;
  int32_t *out = idx + (int64_t)r * k;
  const int tid = threadIdx.x;
  if (n <= k) {
    for (int j = tid; j < k; j += kStreamThreads) out[j] = j < n ? j : -1;
    return;
  }
  const float *row = scores + (int64_t)r * ld;
  const bool vec = (ld & 3) == 0 && ((uintptr_t)scores & 15) == 0;
  int s0, s1;
  stream_segment_of(n, s0, s1);
  // the first batch of the segment goes out with the sample: one memory latency for both
  f32x4 a[kCollectU];
  if (vec) stream_load4(row, s0, s1, a);
  uint32_t lo, hi;
  stream_window(row, n, k, sh, lo, hi);
  uint32_t ca, cc;
  if (vec)
    stream_collect4(row, s0, s1, lo, hi, sh, a, ca, cc);
  else
    stream_collect(row, s0, s1, lo, hi, sh, ca, cc);
  uint32_t ccs[kStreamWaves], c_above, c_cand;
  bool fits;
  stream_counts(ca, cc, sh, ccs, c_above, c_cand, fits);
  const bool window_ok = fits && c_above < (uint32_t)k && (uint32_t)k <= c_cand;
  auto emit = [&](uint32_t slot, int L, uint32_t) { out[slot] = L; };
  if (window_ok) {
    regions_select_emit(ccs, hi, (uint32_t)k - c_above, (uint32_t)k, sh, emit);
  } else {
    uint32_t T, need_eq, cnt_eq;
    stream_threshold(row, n, k, sh, T, need_eq, cnt_eq);
    stream_emit_row(row, s0, s1, T, need_eq, (uint32_t)k, sh, emit);
  }
}

hipError_t launch_topk_stream(const float *scores, int64_t ld, const int32_t *q_pos, int num_q, int k, int32_t *idx,
                              hipStream_t s) {
  hipLaunchKernelGGL(topk_stream_kernel, dim3(num_q), dim3(kStreamThreads), 0, s, scores, ld, q_pos, num_q, k, idx);
  return hipGetLastError();
}

template <int ITEMS>
static hipError_t launch_rows(const float *scores, int64_t ld, const int32_t *q_pos, int num_q, int k,
                              int32_t *idx, hipStream_t s) {
  hipLaunchKernelGGL(topk_rows_kernel<ITEMS>, dim3(num_q), dim3(kTopkBlock), 0, s, scores, ld, q_pos, k, idx);
  return hipGetLastError();
}

hipError_t launch_topk_rows(const float *scores, int64_t ld, const int32_t *q_pos, int num_q, int k,
                            int32_t *idx, int items, hipStream_t s) {
  switch (items) {
    case 1: return launch_rows<1>(scores, ld, q_pos, num_q, k, idx, s);
    case 2: return launch_rows<2>(scores, ld, q_pos, num_q, k, idx, s);
    case 4: return launch_rows<4>(scores, ld, q_pos, num_q, k, idx, s);
    case 8: return launch_rows<8>(scores, ld, q_pos, num_q, k, idx, s);
    case 16: return launch_rows<16>(scores, ld, q_pos, num_q, k, idx, s);
    case 32: return launch_rows<32>(scores, ld, q_pos, num_q, k, idx, s);
    case 64: return launch_rows<64>(scores, ld, q_pos, num_q, k, idx, s);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------------------------------------
// Windowed chunked form for batches of few rows (decode): each row is split into chunks of `chunk` keys, one
// 16-wave workgroup per chunk, so the batch fills the chip. Every workgroup of a row takes the same sample of
// the row as the streaming form (the runs are read from L2 after the first workgroup) and derives the same lower
// bound lo of the window that holds the k-th best key. Chunk c keeps its keys >= lo in LDS during one pass (one
// region per wave, as in the streaming form's collect step) and writes them, in position order, with their
// count: a few hundred per chunk instead of k. A chunk with more than cap = min(k, chunk) such keys, or more than
// a wave's LDS region holds, writes its own exact top-cap instead (it contains the row's top-k within that chunk
// under the same total order; when the chunk's keys >= lo fit cap but not a wave's region, that top-cap also
// holds keys below lo). The merge pass (one 16-wave workgroup per row) gathers the row's M candidates into LDS, in
// position order, and selects k among those >= lo with one histogram pass over the window (window_select_emit).
// When k or more candidates are >= lo the selection is exact (the row's k-th best key is then >= lo, so every
// kept key is a candidate); otherwise the window missed and the merge selects over the whole row from the scores
// instead (as does a row with too many candidates for LDS, or a window that does not settle the threshold).
constexpr int kWMaxChunks = kStreamThreads;   // one count per merge thread
constexpr int kWMergeCap = kStreamWaves * kCandPerWave;
// The merge runs 16 waves: its steps are short chains of barriers, ballots and per-item loops, and four times
// the waves give each lane a quarter of the candidate items.
constexpr int kMergeWaves = 16;
// The chunk pass: waves per workgroup (its chunk of V * 4 * 64 keys per wave stays in registers).
constexpr int kChunkWaves = 16;

// Pass 1: chunk c of row r writes its candidates at slot (r * n_chunks + c) * cap and their count at
// cnt[r * n_chunks + c]; chunk 0 also writes the window's top at cnt[num_q * n_chunks + r] and its bottom at
// cnt[num_q * (n_chunks + 1) + r]. The chunk (V * 256 keys per wave) is loaded into registers before the window is
// known: wave w holds positions w*V*256 .. (w+1)*V*256 - 1, lane l four consecutive positions per load, so lane
// order within a load is position order.
template <int V, int W>
__global__ __launch_bounds__(W * kWave) void topk_wchunk_kernel(const float *__restrict__ scores, int64_t ld,
                                                                     const int32_t *__restrict__ q_pos, int k,
                                                                     int n_chunks, int cap,
                                                                     uint32_t *__restrict__ cand_key,
                                                                     int32_t *__restrict__ cand_pos,
                                                                     uint32_t *__restrict__ cand_cnt) {
  constexpr int CHUNK = V * 4 * W * kWave, CPW = StreamSharedT<W>::CPW;
  static_assert(V >= 1, "a chunk holds at least one 16-byte load per lane");
  __shared__ StreamSharedT<W> sh;
  const int r = blockIdx.x, c = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int start = c * CHUNK;
  const float *row = scores + (int64_t)r * ld;
  const float *crow = row + start;
  // keys of the chunk within the row's allocation (ld), loaded with q_pos; masked to the row's length below
  const int avail = (int)min((int64_t)CHUNK, ld - start);
  const bool vec = (ld & 3) == 0 && ((uintptr_t)scores & 15) == 0;
  const int wbase = w * V * 4 * kWave;
  // the row length first: the sample loads below depend on it and need not wait behind the chunk's loads
  const int n = q_pos[r] + 1;
  f32x4 x[V];
  if (vec) {
    // ld and the chunk's start are multiples of 4, so a lane's four keys lie all inside the allocation or all
    // past it (avail >= 4): every lane loads, past the end the allocation's last four keys, which are never used
    // (positions past the row's length are masked below, and len <= avail). No branch or use separates the loads
    // from the sample's, so all of them are in flight together.
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const int L = wbase + u * 4 * kWave + 4 * lane;
      x[u] = *(const f32x4 *)(crow + min(L, avail - 4));
    }
  } else {
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const int L = wbase + u * 4 * kWave + 4 * lane;
      x[u].x = L + 0 < avail ? crow[L + 0] : 0.f;
      x[u].y = L + 1 < avail ? crow[L + 1] : 0.f;
      x[u].z = L + 2 < avail ? crow[L + 2] : 0.f;
      x[u].w = L + 3 < avail ? crow[L + 3] : 0.f;
    }
  }
  if (n <= k || start >= n) return;   // the merge pass writes rows with n <= k directly
  const int len = min(CHUNK, n - start);
  uint32_t lo, hi;
  stream_window(row, n, k, sh, lo, hi);
  // keys >= lo of this wave's positions -> its LDS region, in position order
  const int cb = w * CPW;
  uint32_t cc = 0u;
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int L = wbase + u * 4 * kWave + 4 * lane;
    const uint32_t kx[4] = {order_key(x[u].x), order_key(x[u].y), order_key(x[u].z), order_key(x[u].w)};
    uint32_t nc = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) nc += (L + j < len && kx[j] >= lo) ? 1u : 0u;
    uint32_t tot;
    uint32_t slot = cc + lane_prefix8(nc, tot);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (L + j < len && kx[j] >= lo) {
        if (slot < (uint32_t)CPW) {
          sh.cand_key[cb + slot] = kx[j];
          sh.cand_pos[cb + slot] = L + j;
        }
        ++slot;
      }
    }
    cc += tot;
  }
  uint32_t ccs[W], c_above, c_cand;
  bool fits;
  stream_counts(0u, cc, sh, ccs, c_above, c_cand, fits);
  const int64_t dst = ((int64_t)r * n_chunks + c) * cap;
  if (fits && c_cand <= (uint32_t)cap) {
    uint32_t base = 0u;
#pragma unroll
    for (int i = 0; i < W; ++i) base += i < w ? ccs[i] : 0u;
    for (uint32_t i = lane; i < cc; i += kWave) {
      cand_key[dst + base + i] = sh.cand_key[cb + i];
      cand_pos[dst + base + i] = start + sh.cand_pos[cb + i];
    }
  } else {   // the chunk's own exact top-cap, by streaming bucket passes over its scores (rare)
    int s0, s1;
    stream_segment_of<W>(len, s0, s1);
    uint32_t T, need_eq, cnt_eq;
    stream_threshold(crow, len, cap, sh, T, need_eq, cnt_eq);
    stream_emit_row(crow, s0, s1, T, need_eq, (uint32_t)cap, sh, [&](uint32_t slot, int L, uint32_t xk) {
      cand_key[dst + slot] = xk;
      cand_pos[dst + slot] = start + L;
    });
    c_cand = (uint32_t)cap;
  }
  if (tid == 0) {
    cand_cnt[(int64_t)r * n_chunks + c] = c_cand;
    if (c == 0) {   // the window, for the merge
      cand_cnt[(int64_t)gridDim.x * n_chunks + r] = hi;
      cand_cnt[(int64_t)gridDim.x * (n_chunks + 1) + r] = lo;
    }
  }
}

// Pass 2: one workgroup per row selects k among its M candidates (or, when M < k or M exceeds the LDS regions,
// over the whole row).
template <int W>
__global__ __launch_bounds__(W * kWave) void topk_wmerge_kernel(const float *__restrict__ scores, int64_t ld,
                                                                     const int32_t *__restrict__ q_pos, int k,
                                                                     int chunk, int n_chunks, int cap,
                                                                     const uint32_t *__restrict__ cand_key,
                                                                     const int32_t *__restrict__ cand_pos,
                                                                     const uint32_t *__restrict__ cand_cnt,
                                                                     int32_t *__restrict__ idx) {
  constexpr int NT = W * kWave, CPW = StreamSharedT<W>::CPW;
  static_assert(NT >= kWMaxChunks, "one count per thread");
  __shared__ StreamSharedT<W> sh;
  __shared__ uint32_t pre[kWMaxChunks + 1];
  const int r = blockIdx.x, tid = threadIdx.x;
  // the counts and the row's window (written by chunk 0 of this row) are loaded with q_pos (chunks past the
  // row's end are masked once n is known)
  const uint32_t v_raw = tid < n_chunks ? cand_cnt[(int64_t)r * n_chunks + tid] : 0u;
  const uint32_t top = cand_cnt[(int64_t)gridDim.x * n_chunks + r];
  const uint32_t lo = cand_cnt[(int64_t)gridDim.x * (n_chunks + 1) + r];
  const int n = q_pos[r] + 1;
  int32_t *out = idx + (int64_t)r * k;
  if (n <= k) {
    for (int j = tid; j < k; j += NT) out[j] = j < n ? j : -1;
    return;
  }
  const int used = (n + chunk - 1) / chunk;   // <= n_chunks <= kWMaxChunks
  const uint32_t v = tid < used ? v_raw : 0u;
  const uint32_t incl = stream_incl_scan(v, sh);
  if (tid < used) pre[tid + 1] = incl;
  if (tid == 0) pre[0] = 0u;
  __syncthreads();
  const uint32_t M = pre[used];
  const float *row = scores + (int64_t)r * ld;
  auto emit = [&](uint32_t slot, int L, uint32_t) { out[slot] = L; };
  if (M < (uint32_t)k || M > (uint32_t)kWMergeCap) {
    int s0, s1;
    stream_segment_of<W>(n, s0, s1);
    uint32_t T, need_eq, cnt_eq;
    stream_threshold(row, n, k, sh, T, need_eq, cnt_eq);
    stream_emit_row(row, s0, s1, T, need_eq, (uint32_t)k, sh, emit);
    return;
  }
  // candidates -> LDS, flat in position order (chunk order, then order within the chunk); every load is issued
  // before the first store, so the row pays one memory latency
  const int64_t base = (int64_t)r * n_chunks * cap;
  constexpr int PM = (kWMergeCap + NT - 1) / NT;
  uint32_t mk[PM];
  int32_t mp[PM];
#pragma unroll
  for (int u = 0; u < PM; ++u) {
    const uint32_t j = (uint32_t)(u * NT + tid);
    mk[u] = 0u;
    mp[u] = 0;
    if (j < M) {
      int a = 0, b = used;   // chunk of flat entry j: pre[a] <= j < pre[a + 1]
      while (b - a > 1) {
        const int mid = (a + b) >> 1;
        if (pre[mid] <= j) a = mid; else b = mid;
      }
      const int64_t g = base + (int64_t)a * cap + (j - pre[a]);
      mk[u] = cand_key[g];
      mp[u] = cand_pos[g];
    }
  }
#pragma unroll
  for (int u = 0; u < PM; ++u) {
    const uint32_t j = (uint32_t)(u * NT + tid);
    if (j < M) {
      sh.cand_key[j] = mk[u];
      sh.cand_pos[j] = mp[u];
    }
  }
  __syncthreads();
  // the flat array seen as W wave regions of CPW pairs
  uint32_t ccs[W];
#pragma unroll
  for (int i = 0; i < W; ++i) ccs[i] = (uint32_t)min(max((int)M - i * CPW, 0), CPW);
  if (!window_select_emit(ccs, lo, top, (uint32_t)k, sh, emit)) {
    int s0, s1;
    stream_segment_of<W>(n, s0, s1);
    uint32_t T, need_eq, cnt_eq;
    stream_threshold(row, n, k, sh, T, need_eq, cnt_eq);
    stream_emit_row(row, s0, s1, T, need_eq, (uint32_t)k, sh, emit);
  }
}

size_t topk_windowed_ws_bytes(int num_q, int n_chunks, int cap) {
  const size_t pairs = (size_t)num_q * n_chunks * cap;
  return (pairs * 8 + 15) / 16 * 16 + (size_t)num_q * (n_chunks + 2) * 4;   // + counts, + each row's window
}

// One chunk of CHUNK keys per workgroup: V 16-byte loads per lane of kChunkWaves waves.
template <int CHUNK>
static void launch_wchunk(const float *scores, int64_t ld, const int32_t *q_pos, int num_q, int k, int n_chunks,
                          int cap, uint32_t *ck, int32_t *cp, uint32_t *cc, hipStream_t s) {
  constexpr int V = CHUNK / (4 * kChunkWaves * kWave);
  hipLaunchKernelGGL((topk_wchunk_kernel<V, kChunkWaves>), dim3(num_q, n_chunks), dim3(kChunkWaves * kWave), 0, s,
                     scores, ld, q_pos, k, n_chunks, cap, ck, cp, cc);
}

hipError_t launch_topk_windowed(const float *scores, int64_t ld, const int32_t *q_pos, int num_q, int k, int chunk,
                                int n_chunks, void *ws, int32_t *idx, hipStream_t s) {
  if (n_chunks > kWMaxChunks) return hipErrorInvalidValue;
  const int cap = min(k, chunk);
  const size_t pairs = (size_t)num_q * n_chunks * cap;
  uint32_t *ck = static_cast<uint32_t *>(ws);
  int32_t *cp = reinterpret_cast<int32_t *>(ck + pairs);
  uint32_t *cc = reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(ws) + (pairs * 8 + 15) / 16 * 16);
  switch (chunk) {
    case 4096: launch_wchunk<4096>(scores, ld, q_pos, num_q, k, n_chunks, cap, ck, cp, cc, s); break;
    case 8192: launch_wchunk<8192>(scores, ld, q_pos, num_q, k, n_chunks, cap, ck, cp, cc, s); break;
    case 16384: launch_wchunk<16384>(scores, ld, q_pos, num_q, k, n_chunks, cap, ck, cp, cc, s); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_wmerge_kernel<kMergeWaves>, dim3(num_q), dim3(kMergeWaves * kWave), 0, s, scores, ld, q_pos,
                     k, chunk, n_chunks, cap, ck, cp, cc, idx);
  return hipGetLastError();
}

hipError_t launch_topk_merge(const int32_t *q_pos, int num_q, int k, int chunk, int n_chunks, const uint32_t *cand_key,
                             const int32_t *cand_pos, int32_t *idx, hipStream_t s) {
  int items = 1;
  while (items * kTopkBlock < n_chunks * k) items <<= 1;
  switch (items) {
#define DSA_MERGE(I) \
  case I: hipLaunchKernelGGL(topk_merge_kernel<I>, dim3(num_q), dim3(kTopkBlock), 0, s, q_pos, k, chunk, n_chunks, \
                             cand_key, cand_pos, idx); break;
    DSA_MERGE(1) DSA_MERGE(2) DSA_MERGE(4) DSA_MERGE(8) DSA_MERGE(16) DSA_MERGE(32) DSA_MERGE(64)
#undef DSA_MERGE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dsa

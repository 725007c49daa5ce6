// Lightning-indexer scores for DSA on gfx950 bf16 MFMA.
//
//   scores[r, s] = sum_j w[r, j] * ReLU(sigma_s * q_idx[r, j, :] . k_idx[slot(b, s), :]),  s = 0 .. q_pos[r]
//
// Defined by the GLM sparse-attention essay (paragraph on the indexer's ReLU: per-head similarities clipped
// at zero, summed with per-head weights, robust enough to run the keys in FP8) and the "DeepSeek Sparse
// Attention" explainer (sections "Make a shortlist first" and "The lightning indexer": every earlier token
// is scored, and the scores only pick positions).
//
// Mapping. For one query row the dot products form the matrix D = Q_r (H_I x d_I) * K^T (d_I x keys), a
// dense contraction, computed with v_mfma_f32_32x32x16_bf16 tiles: heads on M, keys on N, d_I on K. A wave
// keeps its row's Q fragments in registers for the whole key loop; key tiles are staged once per workgroup
// in LDS and shared by the workgroup's rows. The epilogue runs on the accumulator registers: each lane holds
// 16 heads of one key column per tile, so ReLU, the w-weighting and the head sum are in-lane FMAs, and one
// cross-lane add joins the two half-waves. The causal mask is applied by never scoring s > p: key tiles past
// a row's position are skipped and the diagonal tile's store is predicated.
//
// FP8 keys (OCP E4M3) are up-converted exactly to bf16 in registers; since sigma_s > 0,
// ReLU(sigma_s * x) = sigma_s * ReLU(x), so sigma_s multiplies the finished head sum.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "topk_select.h"

namespace dsa {

// ReLU as one v_med3_f32: median(x, 0, FLT_MAX) = max(x, 0) for every finite x (fmaxf would add a
// canonicalising max per element under IEEE NaN rules, and with +inf as the bound the compiler turns the
// median back into that max). A dot product that overflowed to +inf would be clamped to FLT_MAX.
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.40282347e38f); }

template <int HI, int DI, bool FP8, int ROWS, int NW>
struct IndexerCfg {
  static constexpr int MT = (HI + 31) / 32;                      // 32-head M tiles
  static constexpr int KS = DI / 16;                             // K steps of the 32x32x16 MFMA
  static constexpr int WPR = NW / ROWS;                          // waves sharing one row
  static constexpr int BK = 32 * (WPR > 4 ? WPR : 4);            // keys staged per block
  static constexpr int GROUPS = BK / 32;                         // 32-key groups per block
  static constexpr int GPW = GROUPS / WPR;                       // groups per wave per block
  static constexpr int ROW_BYTES = FP8 ? DI : 2 * DI;            // bytes of one key in HBM
  static constexpr int KSTRIDE = FP8 ? DI + 8 : 2 * DI + 16;     // padded LDS row (conflict-free reads)
  static constexpr int CPK = ROW_BYTES / 16;                     // 16-byte chunks per key
  static_assert(DI % 16 == 0 && NW % ROWS == 0 && GROUPS % WPR == 0, "indexer tiling");
};

template <int HI, int DI, bool FP8, int ROWS, int NW>
__global__ __launch_bounds__(NW * kWave) void indexer_kernel(IndexerArgs a, int blocks_per_chunk, int row_blocks) {
  using C = IndexerCfg<HI, DI, FP8, ROWS, NW>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[C::BK * C::KSTRIDE];
  __shared__ float lds_sig[C::BK];
  __shared__ const uint8_t *lds_row[C::BK];  // address of each staged key row, nullptr = past the segment

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  // heavy row blocks (late positions, most keys) first
  const int rb = row_blocks - 1 - (int)blockIdx.x;
  const int r0 = rb * ROWS;
  const int my_slot = wv % ROWS;      // which row of the block this wave serves
  const int my_part = wv / ROWS;      // which share of the key groups
  const int my_row = r0 + my_slot;
  const bool row_ok = my_row < a.num_q;
  const int my_p = row_ok ? a.q_pos[my_row] : -1;
  const int my_seq = row_ok ? a.q_seq[my_row] : -1;

  // this wave's row: Q fragments (A operand, heads x d) and the weights of the heads its lanes accumulate
  bf16x8 qf[C::MT][C::KS];
  float wr[C::MT][16];
#pragma unroll
  for (int t = 0; t < C::MT; ++t) {
    const int head = t * 32 + n;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok && head < HI)
        v = *(const u32x4 *)((const uint16_t *)a.q_idx + ((int64_t)my_row * HI + head) * DI + s * 16 + g * 8);
      qf[t][s] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = t * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
      wr[t][i] = (row_ok && h < HI) ? a.w[(int64_t)my_row * HI + h] : 0.f;
    }
  }

  // rows of one sequence share staged keys; a block straddling sequences runs one segment per sequence
  int seg = 0;
  while (seg < ROWS && r0 + seg < a.num_q) {
    const int b = a.q_seq[r0 + seg];
    int seg_end = seg + 1;
    int p_max = a.q_pos[r0 + seg];
    while (seg_end < ROWS && r0 + seg_end < a.num_q && a.q_seq[r0 + seg_end] == b) {
      p_max = max(p_max, a.q_pos[r0 + seg_end]);
      ++seg_end;
    }
    const bool active = row_ok && my_seq == b && my_slot >= seg && my_slot < seg_end;
    const int kb_lo = blockIdx.y * blocks_per_chunk;
    const int kb_hi = min(kb_lo + blocks_per_chunk, p_max / C::BK + 1);
    for (int kb = kb_lo; kb < kb_hi; ++kb) {
      // ---- stage BK keys: row addresses first (page-table lookups), then 16-byte chunks coalesced per row
      for (int kk = tid; kk < C::BK; kk += NW * kWave) {
        const int s = kb * C::BK + kk;
        const uint8_t *row = nullptr;
        float sig = 0.f;
        if (s <= p_max) {
          const int64_t slot = a.slot(b, s);
          row = (const uint8_t *)a.k_idx + slot * C::ROW_BYTES;
          if constexpr (FP8) sig = a.k_scale[slot];
        }
        lds_row[kk] = row;
        if constexpr (FP8) lds_sig[kk] = sig;
      }
      __syncthreads();
      {
        constexpr int PER = (C::BK * C::CPK + NW * kWave - 1) / (NW * kWave);
        const int tid_l = opaque(tid);
        u32x4 v[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const int c = tid_l + j * NW * kWave;
          const int kk = c / C::CPK, part = c - kk * C::CPK;
          v[j] = u32x4{0u, 0u, 0u, 0u};
          if (c < C::BK * C::CPK) {
            const uint8_t *row = lds_row[kk];
            if (row != nullptr) v[j] = load_global_16(row + part * 16);
          }
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const int c = tid_l + j * NW * kWave;
          if (c >= C::BK * C::CPK) continue;
          const int kk = c / C::CPK, part = c - kk * C::CPK;
          if constexpr (C::KSTRIDE % 16 == 0) {
            *(u32x4 *)(lds_k + kk * C::KSTRIDE + part * 16) = v[j];
          } else {  // 8-byte aligned rows: two 8-byte LDS writes
            *(u32x2 *)(lds_k + kk * C::KSTRIDE + part * 16) = u32x2{v[j].x, v[j].y};
            *(u32x2 *)(lds_k + kk * C::KSTRIDE + part * 16 + 8) = u32x2{v[j].z, v[j].w};
          }
        }
      }
      __syncthreads();
      if (active) {
#pragma unroll
        for (int gi = 0; gi < C::GPW; ++gi) {
          const int grp = my_part * C::GPW + gi;
          const int s0 = kb * C::BK + grp * 32;
          if (s0 > my_p) continue;  // wave-uniform: the whole group is beyond this row
          f32x16 acc[C::MT];
#pragma unroll
          for (int t = 0; t < C::MT; ++t) acc[t] = f32x16{};
          const uint8_t *krow = lds_k + (grp * 32 + n) * C::KSTRIDE;
#pragma unroll
          for (int s = 0; s < C::KS; ++s) {
            bf16x8 bfr;
            if constexpr (FP8) {
              const u32x2 raw = *(const u32x2 *)(krow + s * 16 + g * 8);
              const u32x2 lo = fp8x4_to_bf16x4(raw.x), hi = fp8x4_to_bf16x4(raw.y);
              const u32x4 v = {lo.x, lo.y, hi.x, hi.y};
              bfr = __builtin_bit_cast(bf16x8, v);
            } else {
              bfr = __builtin_bit_cast(bf16x8, *(const u32x4 *)(krow + s * 32 + g * 16));
            }
#pragma unroll
            for (int t = 0; t < C::MT; ++t)
              acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[t][s], bfr, acc[t], 0, 0, 0);
          }
          float part = 0.f;
#pragma unroll
          for (int t = 0; t < C::MT; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) part = fmaf(wr[t][i], relu(acc[t][i]), part);
          part = xor32_sum(part);   // own + other half-wave (v_permlane32_swap)
          const int s = s0 + n;
          if (g == 0 && s <= my_p) {
            if constexpr (FP8) part *= lds_sig[grp * 32 + n];
            a.scores[(int64_t)my_row * a.ld + s] = part;
          }
        }
      }
      __syncthreads();
    }
    seg = seg_end;
  }
}

// The same product with the key tiles streamed into LDS by a dedicated producer wave. Wave NW issues every
// 16-byte global->LDS load of a tile (three tiles in flight) and is the only wave that waits on vector-memory
// counts, so the compute waves' score stores never delay a tile. Rows keep their natural 1 KB-contiguous layout
// in LDS with the 16-byte chunks of key row kk XOR-swizzled by kk, which keeps the MFMA operand reads free of
// bank conflicts without padding. Paged caches (pages of at least RPL rows) take the same loads: the rows of one
// load lie in one page, whose id the producer reads with a scalar load and keeps in LDS for the scale lookups.
template <int HI, int DI, bool FP8, int ROWS, int NW>
struct PipeCfg {
  using B = IndexerCfg<HI, DI, FP8, ROWS, NW>;
  static constexpr int NBUF = 3;
  static constexpr int TILE = B::BK * B::ROW_BYTES;           // bytes of one staged key block
  static constexpr int LOADS = TILE / (kWave * 16);          // wave-wide 1 KB loads per tile
  static constexpr int RPL = kWave / B::CPK;                  // key rows per load
  static constexpr int NV = RPL >= B::CPK ? 1 : B::CPK / RPL; // loads after which the swizzle pattern repeats
  // usable when a tile is whole 1 KB loads, a vmcnt wait can cover one tile, and three tiles fit in LDS
  static constexpr bool OK = TILE % (kWave * 16) == 0 && LOADS < 64 && NBUF * TILE <= 128 * 1024;
  __device__ static __forceinline__ int swz(int chunk, int kk) { return chunk ^ (kk & (B::CPK - 1)); }
};

// Balanced split of a batch of few rows per sequence (decode): the key blocks of every row block (row block rb
// has p_max(rb) / BK + 1 of them, p_max the largest position of its rows) are cut into chunks of
// bpc blocks, ceil(nb / bpc) chunks per row block, and workgroup u takes the u-th chunk in row-block order, so a
// long sequence gets proportionally more workgroups than a short one. bpc is the smallest count from
// ceil(total / target) up that makes at most `target` chunks in all. Every wave computes the same split from
// q_pos; false for a workgroup past the last chunk.
template <int ROWS, int BK>
__device__ __forceinline__ int row_block_nblocks(const IndexerArgs &a, int r) {
  int p = -1;
#pragma unroll
  for (int i = 0; i < ROWS; ++i) {
    const int row = r * ROWS + i;
    if (row < a.num_q) p = max(p, a.q_pos[row]);
  }
  return p < 0 ? 0 : p / BK + 1;
}

// nb0: this lane's row block's block count (row block `lane`; 0 past the last), which the caller loads: the
// block counts of the first 64 row blocks stay in a register (a decode batch rarely has more), so the passes
// below pay one load latency, not one each; the wave reductions and scans run on DPP
template <int ROWS, int BK>
__device__ __forceinline__ bool balanced_unit(const IndexerArgs &a, int row_blocks, int target, int u, int nb0,
                                              int &rb, int &c, int &bpc) {
  const int lane = threadIdx.x & 63;
  auto nblocks = [&](int r) { return row_block_nblocks<ROWS, BK>(a, r); };
  auto nb_of = [&](int base) {
    const int r = base + lane;
    return base == 0 ? nb0 : (r < row_blocks ? nblocks(r) : 0);
  };
  int total = 0, nb_max = 0;
  for (int base = 0; base < row_blocks; base += kWave) {
    const int nb = nb_of(base);
    total += (int)wave_total_sum((uint32_t)nb);
    nb_max = max(nb_max, (int)wave_total_max((uint32_t)nb));
  }
  auto chunks_for = [&](int b) {   // non-increasing in b
    int ch = 0;
    for (int base = 0; base < row_blocks; base += kWave) ch += (int)wave_total_sum((uint32_t)((nb_of(base) + b - 1) / b));
    return ch;
  };
  // ceil(total / target) blocks per chunk can still leave a few more than `target` chunks (each row block rounds
  // up), and those would run as a second round of workgroups after the first: take the smallest bpc that fits,
  // by bisection up to nb_max (one chunk per row block, the fewest there can be)
  int b_lo = max(1, (total + target - 1) / target);
  bpc = b_lo;
  if (b_lo < nb_max && chunks_for(b_lo) > target) {
    int b_hi = nb_max;   // chunks_for(b_lo) > target; b_hi fits, or nothing does
    while (b_hi - b_lo > 1) {
      const int mid = (b_lo + b_hi) / 2;
      if (chunks_for(mid) <= target) b_hi = mid; else b_lo = mid;
    }
    bpc = b_hi;
  }
  int before = 0;
  for (int base = 0; base < row_blocks; base += kWave) {
    const int r = base + lane;
    const int ch = (nb_of(base) + bpc - 1) / bpc;
    const int incl = (int)wave_incl_sum((uint32_t)ch);
    const uint64_t m = ballot(ch > 0 && u >= before + incl - ch && u < before + incl);
    if (m != 0) {
      const int src = __ffsll((unsigned long long)m) - 1;   // wave-uniform
      rb = __builtin_amdgcn_readlane(r, src);
      c = u - (before + __builtin_amdgcn_readlane(incl - ch, src));
      return true;
    }
    before += __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  return false;
}

template <int HI, int DI, bool FP8, int ROWS, int NW, bool PAGED>
__global__ __launch_bounds__((NW + 1) * kWave) void indexer_pipe_kernel(IndexerArgs a, int blocks_per_chunk,
                                                                         int row_blocks, int balance_target) {
  using C = IndexerCfg<HI, DI, FP8, ROWS, NW>;
  using P = PipeCfg<HI, DI, FP8, ROWS, NW>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[P::NBUF * P::TILE];
  __shared__ int32_t lds_page[P::NBUF][P::LOADS];   // paged caches: the page of each load of a tile

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wv == NW;
  const int n = lane & 31, g = lane >> 5;
  int rb, kb_base, bpc;
  if (balance_target > 0) {
    int c;
    const int nb0 = lane < row_blocks ? row_block_nblocks<ROWS, C::BK>(a, lane) : 0;
    if (!balanced_unit<ROWS, C::BK>(a, row_blocks, balance_target, (int)blockIdx.x, nb0, rb, c, bpc)) return;
    rb = __builtin_amdgcn_readfirstlane(rb);   // wave-uniform values: keep them (and the addresses) scalar
    c = __builtin_amdgcn_readfirstlane(c);
    bpc = __builtin_amdgcn_readfirstlane(bpc);
    kb_base = c * bpc;
  } else {
    rb = row_blocks - 1 - (int)blockIdx.x;   // heavy row blocks (late positions, most keys) first
    bpc = blocks_per_chunk;
    kb_base = (int)blockIdx.y * bpc;
  }
  const int r0 = rb * ROWS;
  const int my_slot = wv % ROWS;
  const int my_part = wv / ROWS;
  const int my_row = r0 + my_slot;
  const bool row_ok = !producer && my_row < a.num_q;
  const int my_p = row_ok ? a.q_pos[my_row] : -1;
  const int my_seq = row_ok ? a.q_seq[my_row] : -1;
  constexpr bool paged = PAGED;
  const int shift = a.slot.page_shift;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds_k;
  const int q_ld = lane / C::CPK;   // producer lanes: key row within a load, and the NV chunk offsets
  int coff[P::NV];
#pragma unroll
  for (int v = 0; v < P::NV; ++v)
    coff[v] = opaque(P::swz(lane % C::CPK, v * P::RPL + q_ld) * 16);

  bf16x8 qf[C::MT][C::KS];
  float wr[C::MT][16];
#pragma unroll
  for (int t = 0; t < C::MT; ++t) {
    const int head = t * 32 + n;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok && head < HI)
        v = *(const u32x4 *)((const uint16_t *)a.q_idx + ((int64_t)my_row * HI + head) * DI + s * 16 + g * 8);
      qf[t][s] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = t * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
      wr[t][i] = (row_ok && h < HI) ? a.w[(int64_t)my_row * HI + h] : 0.f;
    }
  }

  int seg = 0;
  while (seg < ROWS && r0 + seg < a.num_q) {
    const int b = a.q_seq[r0 + seg];
    int seg_end = seg + 1;
    int p_max = a.q_pos[r0 + seg];
    while (seg_end < ROWS && r0 + seg_end < a.num_q && a.q_seq[r0 + seg_end] == b) {
      p_max = max(p_max, a.q_pos[r0 + seg_end]);
      ++seg_end;
    }
    const bool active = row_ok && my_seq == b && my_slot >= seg && my_slot < seg_end;
    const int kb_lo = kb_base;
    const int kb_hi = min(kb_lo + bpc, p_max / C::BK + 1);
    const uint8_t *kbase = (const uint8_t *)a.k_idx;
    const int64_t seq0 = (int64_t)b * a.slot.seq_stride;   // contiguous: slot of position 0
    const int32_t *ptab = paged ? a.slot.page_table + (int64_t)b * a.slot.max_pages : nullptr;
    // producer: tile kb into buffer kb % NBUF; keys past p_max load key p_max (never scored). Load j fills key
    // rows j*RPL .. j*RPL+RPL-1 of the tile; lane (q, pc) writes chunk pc of row j*RPL + q, fetching logical
    // chunk swz(pc, row). The swizzle repeats every NV loads, so a lane needs only NV source offsets. For a paged
    // cache the page ids of all the tile's loads are read first (scalar loads, one wait), then the loads go out.
    auto issue = [&](int kb) {
      const int buf = kb % P::NBUF;
      const uint32_t dst = lds_base + (uint32_t)(buf * P::TILE);
      int32_t pg[P::LOADS];
      if constexpr (paged) {
#pragma unroll
        for (int j = 0; j < P::LOADS; ++j) pg[j] = ptab[min(kb * C::BK + j * P::RPL, p_max) >> shift];
        if (lane == 0) {
#pragma unroll
          for (int j = 0; j < P::LOADS; ++j) lds_page[buf][j] = pg[j];
        }
      }
#pragma unroll
      for (int j = 0; j < P::LOADS; ++j) {
        const int s = min(kb * C::BK + j * P::RPL + q_ld, p_max);
        uint64_t src;
        if constexpr (paged)
          src = (uint64_t)(kbase + (((int64_t)pg[j] << shift) + (s & ((1 << shift) - 1))) * C::ROW_BYTES + coff[j % P::NV]);
        else
          src = (uint64_t)(kbase + (seq0 + s) * C::ROW_BYTES + coff[j % P::NV]);
        load_lds_16(src, dst + (uint32_t)(j * kWave * 16));
      }
    };
    if (kb_lo < kb_hi) {
      if (producer) {
        issue(kb_lo);
        if (kb_lo + 1 < kb_hi) issue(kb_lo + 1);
      }
      for (int kb = kb_lo; kb < kb_hi; ++kb) {
        if (producer) {
          // tile kb has landed once at most tile kb+1's loads are outstanding (loads complete in order)
          if (kb + 1 < kb_hi) wait_vmcnt<(P::LOADS < 64 ? P::LOADS : 0)>(); else wait_vmcnt<0>();
        }
        lds_barrier();  // tile kb (and its page ids) visible to every wave; every wave is done with tile kb-1
        if (producer) {
          if (kb + 2 < kb_hi) issue(kb + 2);
        } else if (active) {
          const int buf = kb % P::NBUF;
          const uint8_t *tile = lds_k + buf * P::TILE;
#pragma unroll 1
          for (int gi = 0; gi < C::GPW; ++gi) {   // one group's accumulators live at a time
            const int grp = my_part * C::GPW + gi;
            const int s0 = kb * C::BK + grp * 32;
            if (s0 > my_p) continue;  // wave-uniform: the whole group is beyond this row
            float sig = 1.f;
            if constexpr (FP8) {
              const int sk = min(s0 + n, my_p);
              if constexpr (paged)
                sig = a.k_scale[((int64_t)lds_page[buf][(sk - kb * C::BK) / P::RPL] << shift) + (sk & ((1 << shift) - 1))];
              else
                sig = a.k_scale[seq0 + sk];
            }
            f32x16 acc[C::MT];
#pragma unroll
            for (int t = 0; t < C::MT; ++t) acc[t] = f32x16{};
            const int kk = grp * 32 + n;
            const uint8_t *krow = tile + kk * C::ROW_BYTES;
#pragma unroll
            for (int s = 0; s < C::KS; ++s) {
              bf16x8 bfr;
              if constexpr (FP8) {
                const u32x2 raw = *(const u32x2 *)(krow + P::swz(s, kk) * 16 + g * 8);
                const u32x2 lo = fp8x4_to_bf16x4(raw.x), hi = fp8x4_to_bf16x4(raw.y);
                const u32x4 v = {lo.x, lo.y, hi.x, hi.y};
                bfr = __builtin_bit_cast(bf16x8, v);
              } else {
                bfr = __builtin_bit_cast(bf16x8, *(const u32x4 *)(krow + P::swz(2 * s + g, kk) * 16));
              }
#pragma unroll
              for (int t = 0; t < C::MT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[t][s], bfr, acc[t], 0, 0, 0);
            }
            float part = 0.f;
#pragma unroll
            for (int t = 0; t < C::MT; ++t)
#pragma unroll
              for (int i = 0; i < 16; ++i) part = fmaf(wr[t][i], relu(acc[t][i]), part);
            part = xor32_sum(part);   // own + other half-wave (v_permlane32_swap)
            const int s = s0 + n;
            if (g == 0 && s <= my_p) a.scores[(int64_t)my_row * a.ld + s] = part * sig;
          }
        }
      }
      lds_barrier();  // the next segment reuses the buffers
    }
    seg = seg_end;
  }
}

// Long prefill over a contiguous bf16 key cache (H_I = 64, d_I = 128). Four waves, one per SIMD, each serve two
// adjacent query rows (A, B) of the workgroup's eight, so every key operand read from LDS feeds four MFMAs (two
// rows x two 32-head tiles). The waves load the key tiles themselves (global->LDS through a buffer resource, two
// 256-key tiles in flight, a quarter of a tile per wave) and software-pipeline each 32-key group: the 16 MFMAs of
// row A issue with the previous group's row-B epilogue (ReLU, w-weighting, head sum and store) and the next
// group's operand reads between them, and the 16 MFMAs of row B then cover row A's epilogue and, in a tile's last
// group, the loads of the tile after next. Score stores go through a buffer resource whose size is the row's
// causal extent, so a store past q_pos is dropped by the hardware and the loop body has no branch.
namespace pf {
constexpr int HI = 64, DI = 128, MT = 2, KS = 8;
constexpr int WAVES = 4, ROWS = 2 * WAVES;
constexpr int BK = 256, GROUPS = BK / 32;         // keys per tile, 32-key groups per tile
constexpr int ROW_BYTES = 2 * DI, CPK = ROW_BYTES / 16;
constexpr int TILE = BK * ROW_BYTES;              // 64 KB
constexpr int NBUF = 2;
constexpr int LOAD_BYTES = kWave * 16;            // one wave-wide 16-byte-per-lane load
constexpr int LOADS = TILE / LOAD_BYTES;          // per tile
constexpr int LPW = LOADS / WAVES;                // issued by each wave, LPW / KS per MFMA pair of a stage
constexpr int RPL = kWave / CPK;                  // key rows per load
constexpr int NV = CPK / RPL;                     // loads after which the chunk swizzle repeats
constexpr int NH = LPW / NV;                      // groups of NV loads per wave (one m0 each)
constexpr int SPG = 2;                            // score stores per wave per group (one per row)
constexpr uint32_t kDropped = 0x40000000u;        // store offset past any row's extent: the store is dropped
static_assert(LPW == 2 * KS && NH * NV == LPW && NV * LOAD_BYTES <= 4096 && NBUF * TILE <= 160 * 1024,
              "prefill indexer tiling");
__device__ __forceinline__ int swz(int chunk, int kk) { return chunk ^ (kk & (CPK - 1)); }

// vmcnt allowed while waiting, at the start of tile i's last group, for tile i+1 of a segment. Every wave
// issues, in order: the LPW loads of tiles 0 and 1 up front, then per group a row-B store (stage A) and a row-A
// store (stage B), and in the last group of tile t the loads of tile t+2 before that group's stage-B store.
// Ops issued after tile i+1's loads: for i = 0 the stores of groups 0..GROUPS-2; otherwise the stage-B store of
// tile i-1's last group and the stores of groups 0..GROUPS-2 of tile i.
template <int I>
struct WaitAt {
  static constexpr int value = I == 0 ? (GROUPS - 1) * SPG : 1 + (GROUPS - 1) * SPG;
};
}  // namespace pf

__global__ __launch_bounds__(pf::WAVES * kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void indexer_prefill_kernel(IndexerArgs a, int blocks_per_chunk, int row_blocks) {
  using namespace pf;
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[NBUF * TILE];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, g = lane >> 5;
  const int rb = row_blocks - 1 - (int)blockIdx.x;   // heavy row blocks (late positions, most keys) first
  const int r0 = rb * ROWS;
  const int slotA = 2 * wv, slotB = slotA + 1;
  const int rowA = r0 + slotA, rowB = r0 + slotB;
  const bool okA = rowA < a.num_q, okB = rowB < a.num_q;
  const int pA = okA ? a.q_pos[rowA] : -1, pB = okB ? a.q_pos[rowB] : -1;
  const int seqA = okA ? a.q_seq[rowA] : -1, seqB = okB ? a.q_seq[rowB] : -1;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds_k;

  // loader role of every lane: load jj = NV*h + v of this wave's share (tile load j = wv*LPW + jj) fills chunk pc
  // of key row j*RPL + q_ld with logical chunk swz(pc, row); the swizzle repeats every NV loads, so the source
  // offsets within a tile are per-lane constants, and the LDS side advances with m0 (per h) and the immediate
  // offset v * LOAD_BYTES, which the hardware adds to both addresses
  const int q_ld = lane / CPK;
  uint32_t vo[NH][NV];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int v = 0; v < NV; ++v)
      vo[h][v] = (uint32_t)opaque((wv * LPW + h * NV) * LOAD_BYTES + q_ld * ROW_BYTES +
                                  swz(lane % CPK, v * RPL + q_ld) * 16);
  // consumer role: byte offset of this lane's operand chunk for K-step s within a 32-key group (key n)
  int boff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) boff[s] = opaque(n * ROW_BYTES + swz(2 * s + g, n) * 16);
  // score store offsets: lanes of the upper half-wave hold the same sums and are dropped
  const uint32_t voff = (uint32_t)n * 4u + (g ? kDropped : 0u);

  bf16x8 qa[MT][KS], qb[MT][KS];
  float wa[MT][16], wb[MT][16];
  auto load_row = [&](int row, bool ok, bf16x8 (&qf)[MT][KS], float (&wr)[MT][16]) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int head = t * 32 + n;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (ok) v = *(const u32x4 *)((const uint16_t *)a.q_idx + ((int64_t)row * HI + head) * DI + s * 16 + g * 8);
        qf[t][s] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int h = t * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
        wr[t][i] = ok ? a.w[(int64_t)row * HI + h] : 0.f;
      }
    }
  };
  load_row(rowA, okA, qa, wa);
  load_row(rowB, okB, qb, wb);
  wait_vmcnt<0>();   // the row operands are in registers before any tile load is counted

  const f32x16 zero = {};
  int seg = 0;
  while (seg < ROWS && r0 + seg < a.num_q) {
    const int b = a.q_seq[r0 + seg];
    int seg_end = seg + 1;
    int p_max = a.q_pos[r0 + seg];
    while (seg_end < ROWS && r0 + seg_end < a.num_q && a.q_seq[r0 + seg_end] == b) {
      p_max = max(p_max, a.q_pos[r0 + seg_end]);
      ++seg_end;
    }
    const bool inA = okA && seqA == b && slotA >= seg && slotA < seg_end;
    const bool inB = okB && seqB == b && slotB >= seg && slotB < seg_end;
    // a row outside this segment gets an empty store range: its scores for another sequence's keys are dropped
    const __amdgpu_buffer_rsrc_t rsA =
        __builtin_amdgcn_make_buffer_rsrc(a.scores + (int64_t)(okA ? rowA : 0) * a.ld, (short)0, inA ? (pA + 1) * 4 : 0,
                                          0x00020000);
    const __amdgpu_buffer_rsrc_t rsB =
        __builtin_amdgcn_make_buffer_rsrc(a.scores + (int64_t)(okB ? rowB : 0) * a.ld, (short)0, inB ? (pB + 1) * 4 : 0,
                                          0x00020000);
    const int kb_lo = blockIdx.y * blocks_per_chunk;
    const int kb_hi = min(kb_lo + blocks_per_chunk, p_max / BK + 1);
    const int nt = kb_hi - kb_lo;
    const uint8_t *kseq = (const uint8_t *)a.k_idx + (int64_t)b * a.slot.seq_stride * ROW_BYTES;
    // The buffer resource of tile kb ends at key p_max: keys past it read as zero (they are never scored), no load
    // leaves the sequence's cache, and a tile past the segment's last loads nothing but zeros.
    auto tile_rsrc = [&](int kb) {
      const int64_t first = (int64_t)kb * BK;
      return raw_rsrc(kseq + first * ROW_BYTES, (uint32_t)max(0, (int)(p_max + 1 - first)) * ROW_BYTES);
    };
    auto tile_m0 = [&](int kb) { return lds_base + (uint32_t)((kb % NBUF) * TILE + wv * LPW * LOAD_BYTES); };
    auto load_one = [&](const u32x4 &rs, uint32_t m0, int jj) {
      const uint32_t mh = m0 + (uint32_t)((jj / NV) * NV * LOAD_BYTES);
      switch (jj % NV) {
        case 0: load_lds_16_buf<0 * LOAD_BYTES>(rs, vo[jj / NV][0], mh); break;
        case 1: load_lds_16_buf<1 * LOAD_BYTES>(rs, vo[jj / NV][1], mh); break;
        case 2: load_lds_16_buf<2 * LOAD_BYTES>(rs, vo[jj / NV][2], mh); break;
        default: load_lds_16_buf<3 * LOAD_BYTES>(rs, vo[jj / NV][3], mh); break;
      }
    };
    auto issue = [&](int kb) {
      const u32x4 rs = tile_rsrc(kb);
      const uint32_t m0 = tile_m0(kb);
#pragma unroll
      for (int jj = 0; jj < LPW; ++jj) load_one(rs, m0, jj);
    };
    if (nt > 0) {
      issue(kb_lo);
      if (nt > 1) issue(kb_lo + 1);
      if (nt > 1) wait_vmcnt<LPW>(); else wait_vmcnt<0>();
      lds_barrier();   // tile kb_lo visible to every wave

      bf16x8 bc[KS], bn[KS];
      {
        const uint8_t *tile = lds_k + (kb_lo % NBUF) * TILE;
#pragma unroll
        for (int s = 0; s < KS; ++s) bc[s] = *(const bf16x8 *)(tile + boff[s]);
      }
      f32x16 accA[MT], accB[MT];
      accB[0] = zero;
      accB[1] = zero;
      int prev_s0 = 1 << 28;   // no previous group yet: its row-B store lands past every extent

      // one software-pipelined stage: the MFMAs of one row (acc <- q x bc) with the epilogue of eacc / ew between
      // them and, by tag, the next group's operand reads (READS) or the loads of tile lkb (LOADS)
      auto stage = [&](auto reads_tag, auto loads_tag, f32x16 (&acc)[MT], const bf16x8 (&qf)[MT][KS],
                       const f32x16 (&eacc)[MT], const float (&ew)[MT][16], const __amdgpu_buffer_rsrc_t &ers,
                       int es0, const uint8_t *ntile, int lkb) {
        constexpr bool READS = decltype(reads_tag)::value;
        constexpr bool LOADS = decltype(loads_tag)::value;
        u32x4 lrs = {0u, 0u, 0u, 0u};
        uint32_t lm0 = 0;
        if constexpr (LOADS) {
          lrs = tile_rsrc(lkb);
          lm0 = tile_m0(lkb);
        }
        float part[4] = {0.f, 0.f, 0.f, 0.f};   // four independent FMA chains
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[0][s], bc[s], s ? acc[0] : zero, 0, 0, 0);
          acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[1][s], bc[s], s ? acc[1] : zero, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = (4 * s + e) >> 4, i = (4 * s + e) & 15;
            part[e] = fmaf(ew[t][i], relu(eacc[t][i]), part[e]);
          }
          if constexpr (READS) bn[s] = *(const bf16x8 *)(ntile + boff[s]);
          if constexpr (LOADS) {
            load_one(lrs, lm0, 2 * s);
            load_one(lrs, lm0, 2 * s + 1);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          if constexpr (READS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          if constexpr (LOADS) __builtin_amdgcn_sched_barrier(0);   // two loads per MFMA pair, not bunched
        }
        const float tot = xor32_sum((part[0] + part[1]) + (part[2] + part[3]));
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), ers, voff + (uint32_t)es0 * 4u, 0, 0);
      };

      for (int kb = kb_lo; kb < kb_hi; ++kb) {
        const int i = kb - kb_lo;
        const uint8_t *tile = lds_k + (kb % NBUF) * TILE;
#pragma unroll
        for (int gi = 0; gi < GROUPS; ++gi) {
          const int s0 = kb * BK + gi * 32;
          if (gi < GROUPS - 1) {
            const uint8_t *ntile = tile + (gi + 1) * 32 * ROW_BYTES;
            stage(std::true_type{}, std::false_type{}, accA, qa, accB, wb, rsB, prev_s0, ntile, 0);
            stage(std::false_type{}, std::false_type{}, accB, qb, accA, wa, rsA, s0, ntile, 0);
          } else {
            // tile kb+1 landed (own loads, then everyone's via the barrier); every wave is done with tile kb,
            // whose buffer then takes tile kb+2 (loads past the segment fetch zeros and are drained at its end)
            if (i + 1 < nt) {
              if (i == 0) wait_vmcnt<WaitAt<0>::value>(); else wait_vmcnt<WaitAt<1>::value>();
            }
            lds_barrier();
            // past the last tile the operand reads fetch stale, in-bounds LDS that is never used
            const uint8_t *ntile = lds_k + ((kb + 1) % NBUF) * TILE;
            stage(std::true_type{}, std::false_type{}, accA, qa, accB, wb, rsB, prev_s0, ntile, 0);
            stage(std::false_type{}, std::true_type{}, accB, qb, accA, wa, rsA, s0, ntile, kb + 2);
          }
#pragma unroll
          for (int s = 0; s < KS; ++s) bc[s] = bn[s];
          prev_s0 = s0;
        }
      }
      // the last group's row-B epilogue
      {
        float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < MT * 16; ++e) part[e & 3] = fmaf(wb[e >> 4][e & 15], relu(accB[e >> 4][e & 15]), part[e & 3]);
        const float tot = xor32_sum((part[0] + part[1]) + (part[2] + part[3]));
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), rsB, voff + (uint32_t)prev_s0 * 4u, 0, 0);
      }
      wait_vmcnt<0>();  // zero-filled loads past the segment have landed
      lds_barrier();    // the next segment reuses the buffers
    }
    seg = seg_end;
  }
}


// Decode batches (one or two query rows per sequence, H_I = 64, d_I = 128, contiguous or paged caches): every wave
// streams its own run of 32-key tiles from HBM straight into registers, so there is no LDS staging, no producer
// wave and no workgroup barrier between the loads and the MFMAs. The split is the balanced one above at wave
// granularity (one unit = one wave, one block = one 32-key tile), and each wave keeps D tiles of loads in flight
// in a register ring.
//
// The arithmetic is the staged kernels' own: for K step s lane (n, g) feeds the MFMA the 8 key elements
// 16 s + 8 g .. +7 of key n (bf16: bytes 32 s + 16 g .. +15, one 16-byte chunk; FP8: bytes 16 s + 8 g .. +7), the
// accumulators see the steps in the same order, and the epilogue sums the heads in the same order, so every score
// is bit-identical to theirs. Loads: for bf16 keys, load j of lane (n, g) is exactly step j's chunk (2 j + g); for
// FP8 keys, load j of lane (n, g) brings chunk 2 j + g (step 2 j + g, both half-waves' bytes), and one
// v_permlane32_swap per dword pair hands each half-wave the bytes it needs of steps 2 j and 2 j + 1. Lanes n and
// n + 32 read 32 adjacent bytes of key n in every load, and a tile's loads cover its 32 key rows whole.
namespace dk {
constexpr int HI = 64, DI = 128, MT = 2, KS = 8;
}

// One wave's run of 32-key tiles t_lo .. t_lo + nt - 1 of sequence b (keys past p_max load key p_max and are
// never scored) through the MFMAs and epilogues of ROWS rows (Q fragments qf, head weights wr). `operands()` runs
// once the first ring turn of loads is out (a caller loads the rows' Q and w there), and every load has landed
// before the first tile is consumed. emit(t, i, v) receives row i's score v of key 32 t + n in lane (n, g) (both
// half-waves hold it); t = -1 means no tile (the pipeline's start), with nothing to store.
//
// Loads: a ring of D tiles, refilled as soon as a tile is consumed; past the run's end it reloads the last tile,
// so every group of U tiles runs the same straight-line code and the compiler counts the loads in flight exactly
// (the last nt % U tiles follow with their loads already issued). PM = 0: a contiguous cache, the sequence starting
// at slot b * seq_stride. PM = 1 (pages of at least 32 keys, so a tile lies in one page) and PM = 2 (shorter pages):
// the page id (PM = 1: the tile's, one value for the wave; PM = 2: each lane's key's) of the tile a ring slot loads
// next is loaded one ring turn ahead, so the key loads never wait on a page-table lookup. The scheduling fences
// keep the compiler from merging consecutive tiles' MFMAs, which would need several tiles' keys at once.
//
// Software pipeline: the MFMAs of tile t accumulate into one of two accumulator sets while the epilogue of tile
// t - 1 (ReLU, w-weighting, head sum) runs on the other, so the VALU work of one tile overlaps the MFMAs of the
// next; the set's tile index and scale travel with it (the ring slot is reloaded meanwhile).
template <bool FP8, int ROWS, int D, int PM, class Operands, class Emit>
__device__ __forceinline__ void stream_key_tiles(const IndexerArgs &a, int b, int p_max, int t_lo, int nt,
                                                 const bf16x8 (&qf)[ROWS][dk::MT][dk::KS],
                                                 const float (&wr)[ROWS][dk::MT][16], Operands operands, Emit emit) {
  using namespace dk;
  constexpr int ROW_BYTES = FP8 ? DI : 2 * DI;
  constexpr int NLD = ROW_BYTES / 32;   // 16-byte loads per lane per tile
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;
  const uint8_t *kbase = (const uint8_t *)a.k_idx;
  const int shift = a.slot.page_shift;
  const int64_t seq0 = (int64_t)b * a.slot.seq_stride;
  const int32_t *ptab = PM ? a.slot.page_table + (int64_t)b * a.slot.max_pages : nullptr;
  auto page_of = [&](int t) {   // the tile's page (PM = 1) or this lane's key's (PM = 2)
    return ptab[min(t * 32 + (PM == 2 ? n : 0), p_max) >> shift];
  };
  const int t_end = t_lo + nt - 1;   // last tile of the run

  u32x4 kd[D][NLD];
  float sg[D];
  int pgv[D];
  // tile t's loads into ring slot j (key s = min(32 t + n, p_max)), then the page ids of t_next, the tile slot j
  // loads after t
  auto issue = [&](int t, int t_next, int j) {
    const int s = min(t * 32 + n, p_max);
    const uint8_t *rowp;
    const float *scp;
    if constexpr (PM == 2) {
      const int64_t slot = ((int64_t)pgv[j] << shift) + (s & ((1 << shift) - 1));
      rowp = kbase + slot * ROW_BYTES;
      scp = FP8 ? a.k_scale + slot : nullptr;
    } else {
      // one base per tile for the wave (scalar), the key's offset from it in 32 bits
      const int64_t slot0 = PM ? (int64_t)__builtin_amdgcn_readfirstlane(pgv[j]) << shift : seq0;
      const int off = PM ? (s & ((1 << shift) - 1)) : s;
      rowp = kbase + slot0 * ROW_BYTES + (uint32_t)(off * ROW_BYTES);
      scp = FP8 ? a.k_scale + slot0 + off : nullptr;
    }
#pragma unroll
    for (int l = 0; l < NLD; ++l) kd[j][l] = *(const u32x4 *)(rowp + (2 * l + g) * 16);
    if constexpr (FP8) sg[j] = *scp;
    if constexpr (PM != 0) pgv[j] = page_of(t_next);
  };

  f32x16 acc[2][ROWS][MT];
  float sgp[2] = {1.f, 1.f};
  int tp[2] = {-1, -1};
#pragma unroll
  for (int i = 0; i < ROWS; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[1][i][m] = f32x16{};
  auto mfmas = [&](int t, int j, int par) {
#pragma unroll
    for (int i = 0; i < ROWS; ++i)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[par][i][m] = f32x16{};
#pragma unroll
    for (int l = 0; l < NLD; ++l) {
      u32x4 v = kd[j][l];
      if constexpr (FP8) {
        // lanes 0..31 take the partner's first dword pair (step 2l + 1, half 0) in place of their second;
        // lanes 32..63 take the partner's second pair (step 2l, half 1) in place of their first.
        // v_permlane32_swap swaps lanes 32..63 of its first operand with lanes 0..31 of its second.
        const auto x = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
        const auto y = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
        v.x = x[0];
        v.z = x[1];
        v.y = y[0];
        v.w = y[1];
      }
#pragma unroll
      for (int h = 0; h < (FP8 ? 2 : 1); ++h) {
        bf16x8 bfr;
        if constexpr (FP8) {
          const u32x2 lo = fp8x4_to_bf16x4(h ? v.z : v.x), hi = fp8x4_to_bf16x4(h ? v.w : v.y);
          const u32x4 cv = {lo.x, lo.y, hi.x, hi.y};
          bfr = __builtin_bit_cast(bf16x8, cv);
        } else {
          bfr = __builtin_bit_cast(bf16x8, v);
        }
        const int s = FP8 ? 2 * l + h : l;
#pragma unroll
        for (int i = 0; i < ROWS; ++i)
#pragma unroll
          for (int m = 0; m < MT; ++m)
            acc[par][i][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[i][m][s], bfr, acc[par][i][m], 0, 0, 0);
      }
    }
    sgp[par] = FP8 ? sg[j] : 1.f;
    tp[par] = t;
  };
  auto epilogue = [&](int par) {
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
      float part = 0.f;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int e = 0; e < 16; ++e) part = fmaf(wr[i][m][e], relu(acc[par][i][m][e]), part);
      part = xor32_sum(part);   // own + other half-wave
      emit(tp[par], i, part * sgp[par]);
    }
  };

  constexpr int U = D % 2 ? 2 * D : D;   // a whole number of ring turns and of accumulator-set turns
  if constexpr (PM != 0) {
#pragma unroll
    for (int j = 0; j < D; ++j) pgv[j] = page_of(min(t_lo + j, t_end));
  }
#pragma unroll
  for (int j = 0; j < D; ++j) issue(min(t_lo + j, t_end), min(t_lo + j + D, t_end), j);
  operands();
  wait_vmcnt<0>();
  __builtin_amdgcn_sched_barrier(0);
  int i0 = 0;
  for (; i0 + U <= nt; i0 += U) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      mfmas(t_lo + i0 + k, k % D, k % 2);
      epilogue((k + 1) % 2);
      __builtin_amdgcn_sched_barrier(0);
      issue(min(t_lo + i0 + k + D, t_end), min(t_lo + i0 + k + 2 * D, t_end), k % D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int k = 0; k < U - 1; ++k) {
    if (i0 + k < nt) {
      mfmas(t_lo + i0 + k, k % D, k % 2);
      epilogue((k + 1) % 2);
      if (k + D < U - 1 && i0 + k + D < nt)   // a tile of this tail whose slot is not yet loaded
        issue(t_lo + i0 + k + D, t_lo + i0 + k + D, k % D);
    }
  }
  // the last tile's epilogue (tile i of the run used set i % 2)
  if ((nt - 1) % 2) epilogue(1); else epilogue(0);
}

template <bool FP8, int ROWS, int NW, int D, int PM>
__global__ __launch_bounds__(NW * kWave) void indexer_decode_kernel(IndexerArgs a, int row_blocks, int target) {
  using namespace dk;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int n = lane & 31, g = lane >> 5;
  // positions and sequences of the rows of row block `lane` (the first 64 row blocks): the split's block counts,
  // and the wave's own rows by a lane read when its row block is among them
  int qp[ROWS], qs[ROWS];
  int pmax0 = -1;
#pragma unroll
  for (int i = 0; i < ROWS; ++i) {
    const int row = lane * ROWS + i;
    const bool ok = row < a.num_q;
    qp[i] = ok ? a.q_pos[row] : -1;
    qs[i] = ok ? a.q_seq[row] : -1;
    pmax0 = max(pmax0, qp[i]);
  }
  int rb, c, bpc;
  if (!balanced_unit<ROWS, 32>(a, row_blocks, target, (int)blockIdx.x * NW + wv, pmax0 < 0 ? 0 : pmax0 / 32 + 1, rb,
                               c, bpc))
    return;
  rb = __builtin_amdgcn_readfirstlane(rb);
  c = __builtin_amdgcn_readfirstlane(c);
  bpc = __builtin_amdgcn_readfirstlane(bpc);
  const int r0 = rb * ROWS;
  int rpos[ROWS], rseq[ROWS];
#pragma unroll
  for (int i = 0; i < ROWS; ++i) {
    const int row = r0 + i;
    if (rb < kWave) {
      rpos[i] = __builtin_amdgcn_readlane(qp[i], rb);
      rseq[i] = __builtin_amdgcn_readlane(qs[i], rb);
    } else {
      rpos[i] = row < a.num_q ? a.q_pos[row] : -1;
      rseq[i] = row < a.num_q ? a.q_seq[row] : -1;
    }
  }

  // The row operands (Q fragments, head weights) are loaded after the first tiles' loads have gone out, so the
  // two latencies overlap; one full wait then covers both, and the tile loop starts with no load of unknown age
  // in flight (the compiler's waits for the operands would otherwise sit inside the loop and drain the ring).
  bf16x8 qf[ROWS][MT][KS];
  float wr[ROWS][MT][16];
  auto load_rows = [&]() {
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
      const int row = r0 + i;
      const bool ok = row < a.num_q;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (ok) v = *(const u32x4 *)((const uint16_t *)a.q_idx + ((int64_t)row * HI + t * 32 + n) * DI + s * 16 + g * 8);
          qf[i][t][s] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {   // heads t*32 + 8q + 4g .. +3
          f32x4 v = {0.f, 0.f, 0.f, 0.f};
          if (ok) v = *(const f32x4 *)(a.w + (int64_t)row * HI + t * 32 + q * 8 + g * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) wr[i][t][q * 4 + e] = v[e];
        }
      }
    }
  };
  bool rows_loaded = false;

  int seg = 0;
  while (seg < ROWS && r0 + seg < a.num_q) {
    const int b = __builtin_amdgcn_readfirstlane(rseq[seg]);
    int seg_end = seg + 1;
    int p_max = rpos[seg];
    while (seg_end < ROWS && r0 + seg_end < a.num_q && rseq[seg_end] == b) {
      p_max = max(p_max, rpos[seg_end]);
      ++seg_end;
    }
    p_max = __builtin_amdgcn_readfirstlane(p_max);
    // score stores go through one buffer resource per row whose size is the row's causal extent in this segment
    // (zero for a row of another sequence): stores past q_pos are dropped by the hardware, so neither the loop nor
    // the stores branch, and the compiler can count the loads in flight exactly
    __amdgpu_buffer_rsrc_t rs[ROWS];
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
      const bool in = i >= seg && i < seg_end;
      rs[i] = __builtin_amdgcn_make_buffer_rsrc(a.scores + (int64_t)(in ? r0 + i : 0) * a.ld, (short)0,
                                                in ? (rpos[i] + 1) * 4 : 0, 0x00020000);
    }
    const int t_lo = c * bpc;
    const int nt = min(t_lo + bpc, p_max / 32 + 1) - t_lo;
    if (nt > 0) {
      // lanes n < 32 store key t*32 + n; lanes 32..63 hold the same sums and store past every resource's end (the
      // whole offset is in the VGPR operand, which the range check covers; 2^31 + 4 * 2^20 stays below 2^32); tile
      // -1 stores past every end too
      const uint32_t voff = g ? 0x7ffffff0u : (uint32_t)n * 4u;
      stream_key_tiles<FP8, ROWS, D, PM>(
          a, b, p_max, t_lo, nt, qf, wr,
          [&]() {
            if (!rows_loaded) {
              load_rows();
              rows_loaded = true;
            }
          },
          [&](int t, int i, float v) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs[i], voff + (uint32_t)t * 128u, 0, 0);
          });
    }
    seg = seg_end;
  }
}

// Page mode of stream_key_tiles: 0 contiguous, 1 pages of at least one 32-key tile, 2 shorter pages.
static int page_mode(const IndexerArgs &a) {
  return a.slot.page_table == nullptr ? 0 : (a.slot.page_shift >= 5 ? 1 : 2);
}

template <bool FP8, int ROWS, int NW, int D>
static hipError_t launch_decode(const IndexerArgs &a, int target_waves, hipStream_t st) {
  const int row_blocks = (a.num_q + ROWS - 1) / ROWS;
  // the split makes at most max(target, row_blocks) chunks (one per row block when even that exceeds the target)
  const int units = max(target_waves, row_blocks);
  const dim3 grid((units + NW - 1) / NW), block(NW * kWave);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, st, a, row_blocks, target_waves); };
  switch (page_mode(a)) {
    case 0: go(indexer_decode_kernel<FP8, ROWS, NW, D, 0>); break;
    case 1: go(indexer_decode_kernel<FP8, ROWS, NW, D, 1>); break;
    default: go(indexer_decode_kernel<FP8, ROWS, NW, D, 2>); break;
  }
  return hipGetLastError();
}

// Fused indexer -> top-k for decode batches: a workgroup scores one 8192-key chunk of one query row into LDS and
// selects the chunk's top-k there, so the scores never reach HBM; topk_merge_kernel then selects among the
// chunks' candidates. The "Sparse Attention Architecture Evolution" page names fusing the indexer operators as
// the deployment optimisation. Each of the eight waves streams 32 of the chunk's 32-key tiles through registers
// with the decode indexer's own loop (stream_key_tiles), so every score is bit-identical to dsa_indexer_scores'
// for such batches and the selection is the one dsa_topk makes from it; the select is the shared block-wide bucket
// select over 16 keys per thread.
namespace ft {
constexpr int WAVES = 8, NT = WAVES * kWave;
constexpr int KC = 8192;                       // keys of one workgroup
constexpr int TPW = KC / 32 / WAVES;           // 32-key tiles per wave
constexpr int ITEMS = KC / NT;
}  // namespace ft

template <bool FP8, int PM>
__global__ __launch_bounds__(ft::NT) void indexer_topk_kernel(IndexerArgs a, int k, int n_chunks,
                                                              uint32_t *__restrict__ cand_key,
                                                              int32_t *__restrict__ cand_pos) {
  using namespace ft;
  using dk::MT;
  using dk::KS;
  __shared__ float sc[KC];
  __shared__ TopkSharedT<NT> tsh;

  const int r = blockIdx.x, c = blockIdx.y;
  const int b = a.q_seq[r], p = a.q_pos[r], n = p + 1;
  if (n <= k) return;                 // the merge pass writes such rows directly
  const int start = c * KC;
  if (start >= n) return;
  const int len = min(KC, n - start);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nn = lane & 31, g = lane >> 5;
  const int t_lo = start / 32 + wv * TPW;
  const int nt = min(TPW, p / 32 + 1 - t_lo);
  if (nt > 0) {
    bf16x8 qf[1][MT][KS];
    float wr[1][MT][16];
    auto load_row = [&]() {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
          qf[0][t][s] = __builtin_bit_cast(
              bf16x8, *(const u32x4 *)((const uint16_t *)a.q_idx + ((int64_t)r * dk::HI + t * 32 + nn) * dk::DI +
                                       s * 16 + g * 8));
#pragma unroll
        for (int q = 0; q < 4; ++q) {   // heads t*32 + 8q + 4g .. +3
          const f32x4 v = *(const f32x4 *)(a.w + (int64_t)r * dk::HI + t * 32 + q * 8 + g * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) wr[0][t][q * 4 + e] = v[e];
        }
      }
    };
    // scores of this chunk's keys 0 .. len-1 into LDS (tile -1 is the pipeline's start: nothing to store)
    stream_key_tiles<FP8, 1, FP8 ? 3 : 2, PM>(a, b, p, t_lo, nt, qf, wr, load_row, [&](int t, int, float v) {
      const int s = t * 32 + nn;
      if (t >= 0 && g == 0 && s <= p) sc[s - start] = v;
    });
  }
  __syncthreads();
  uint32_t key[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int L = i * NT + tid;
    key[i] = L < len ? order_key(sc[L]) : 0u;
  }
  const int64_t dst = ((int64_t)r * n_chunks + c) * k;
  select_topk<ITEMS, NT>(key, len, k, [&](int rank, int L, uint32_t kv) {
    cand_key[dst + rank] = kv;
    cand_pos[dst + rank] = start + L;
  }, tsh);
}

hipError_t launch_indexer_topk(const IndexerArgs &a, int k, uint32_t *cand_key, int32_t *cand_pos, int32_t *idx,
                               hipStream_t st) {
  if (a.H_I != dk::HI || a.d_I != dk::DI) return hipErrorInvalidValue;
  const int n_chunks = (a.max_kv_len + ft::KC - 1) / ft::KC;
  const dim3 grid(a.num_q, n_chunks), block(ft::NT);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, st, a, k, n_chunks, cand_key, cand_pos); };
  switch (page_mode(a) + (a.fp8 ? 3 : 0)) {
    case 0: go(indexer_topk_kernel<false, 0>); break;
    case 1: go(indexer_topk_kernel<false, 1>); break;
    case 2: go(indexer_topk_kernel<false, 2>); break;
    case 3: go(indexer_topk_kernel<true, 0>); break;
    case 4: go(indexer_topk_kernel<true, 1>); break;
    default: go(indexer_topk_kernel<true, 2>); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_merge(a.q_pos, a.num_q, k, ft::KC, n_chunks, cand_key, cand_pos, idx, st);
}

size_t indexer_topk_ws_bytes(int num_q, int max_kv_len, int k) {
  const int n_chunks = (max_kv_len + ft::KC - 1) / ft::KC;
  return (size_t)num_q * n_chunks * k * 8;
}

// Key-range chunks per row block: enough workgroups to fill the chip when rows are few.
struct Split {
  int chunks, bpc;   // chunks of the key range, key blocks per chunk
};
static Split key_split(int max_kv_len, int bk, int row_blocks, int target_wgs) {
  const int max_blocks = (max_kv_len + bk - 1) / bk;
  int chunks = (target_wgs + row_blocks - 1) / row_blocks;
  chunks = max(1, min(chunks, max_blocks));
  const int bpc = (max_blocks + chunks - 1) / chunks;
  return {(max_blocks + bpc - 1) / bpc, bpc};
}

template <int HI, int DI, bool FP8, int ROWS>
static hipError_t launch_t(const IndexerArgs &a, int target_wgs, hipStream_t st) {
  constexpr int NW = 8;
  using C = IndexerCfg<HI, DI, FP8, ROWS, NW>;
  const int row_blocks = (a.num_q + ROWS - 1) / ROWS;
  if constexpr (HI == pf::HI && DI == pf::DI && !FP8 && ROWS == pf::ROWS) {
    if (a.slot.page_table == nullptr) {
      const Split sp = key_split(a.max_kv_len, pf::BK, row_blocks, target_wgs);
      hipLaunchKernelGGL(indexer_prefill_kernel, dim3(row_blocks, sp.chunks), dim3(pf::WAVES * kWave), 0, st, a,
                         sp.bpc, row_blocks);
      return hipGetLastError();
    }
  }
  if constexpr (HI == dk::HI && DI == dk::DI && ROWS < 8) {
    // decode batches: register-streamed tiles, one wave per unit of the balanced split. One row a wave: two waves
    // a SIMD, three FP8 (two bf16) tiles in the ring; two rows a wave (their Q, w and two accumulator sets): one
    // wave a SIMD, two tiles in the ring (deeper rings spill)
    if constexpr (ROWS == 1) return launch_decode<FP8, 1, 8, FP8 ? 3 : 2>(a, target_wgs * 8, st);
    else return launch_decode<FP8, ROWS, 4, 2>(a, target_wgs * 4, st);
  }
  const Split sp = key_split(a.max_kv_len, C::BK, row_blocks, target_wgs);
  const int chunks = sp.chunks, bpc = sp.bpc;
  if constexpr (PipeCfg<HI, DI, FP8, ROWS, NW>::OK) {
    using P = PipeCfg<HI, DI, FP8, ROWS, NW>;
    // paged caches whose pages hold whole loads (page_size >= RPL); fewer than 8 rows per workgroup (decode):
    // the balanced split, about target_wgs workgroups in all
    const bool paged = a.slot.page_table != nullptr;
    if (!paged || (1 << a.slot.page_shift) >= P::RPL) {
      auto kern = paged ? indexer_pipe_kernel<HI, DI, FP8, ROWS, NW, true> : indexer_pipe_kernel<HI, DI, FP8, ROWS, NW, false>;
      if (ROWS < 8) {
        hipLaunchKernelGGL(kern, dim3(target_wgs + row_blocks), dim3((NW + 1) * kWave), 0, st, a, 0, row_blocks,
                           target_wgs);
      } else {
        hipLaunchKernelGGL(kern, dim3(row_blocks, chunks), dim3((NW + 1) * kWave), 0, st, a, bpc, row_blocks, 0);
      }
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((indexer_kernel<HI, DI, FP8, ROWS, NW>), dim3(row_blocks, chunks), dim3(NW * kWave), 0, st, a,
                     bpc, row_blocks);
  return hipGetLastError();
}

template <int HI, int DI, bool FP8>
static hipError_t launch_rows(const IndexerArgs &a, int rows_per_wg, int target_wgs, hipStream_t st) {
  switch (rows_per_wg) {
    case 1: return launch_t<HI, DI, FP8, 1>(a, target_wgs, st);
    case 2: return launch_t<HI, DI, FP8, 2>(a, target_wgs, st);
    case 8: return launch_t<HI, DI, FP8, 8>(a, target_wgs, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_indexer(const IndexerArgs &a, int rows_per_wg, int target_wgs, hipStream_t st) {
  if (a.H_I == 64 && a.d_I == 128)
    return a.fp8 ? launch_rows<64, 128, true>(a, rows_per_wg, target_wgs, st)
                 : launch_rows<64, 128, false>(a, rows_per_wg, target_wgs, st);
  if (a.H_I == 4 && a.d_I == 32)
    return a.fp8 ? launch_rows<4, 32, true>(a, rows_per_wg, target_wgs, st)
                 : launch_rows<4, 32, false>(a, rows_per_wg, target_wgs, st);
  return hipErrorInvalidValue;
}

}  // namespace dsa

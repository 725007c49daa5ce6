// Sparse MQA attention for DSA on gfx950: exact softmax over the gathered top-k latent rows.
//
//   z_i = sm_scale * q[r, h, :] . c_i,   out[r, h, :] = sum_i softmax(z)_i * c_i[0:D_v],   lse[r, h] = log sum_i e^{z_i}
//   over the rows c_i = latent[slot(b, idx[r, i])] with idx[r, i] != -1.
//
// Defined by the GLM sparse-attention essay: the softmax over the survivors is exact with the real values
// (paragraph on the sparse-attention bet); MLA caches one latent per token and, with the up-projections
// absorbed, every head scores against that same latent, so one gathered row serves all heads (paragraphs
// on MLA's absorbed read); gathering the scattered rows is the engineering problem (paragraph on decode
// and the gather kernels). "DeepSeek Sparse Attention" explainer, section "Indexing and main attention are
// separate": the indexer picks positions, attention computes the weights.
//
// Mapping (a workgroup = one query row x 128 heads, one wave per 32 heads, one wave per SIMD; every head of
// the workgroup shares each gathered row):
//   prologue every selected row's address is resolved once (index list and page table) into LDS;
//   gather  32 rows per tile go straight from HBM into LDS with 16-byte global_load_lds (no register
//           staging), three tiles in flight, so the gather of tile t+2 overlaps the math of tile t;
//   layout  a tile keeps each 1152-byte row contiguous; the 16-byte chunks of a row are XOR-swizzled so that
//           both LDS reads below are free of bank conflicts;
//   QK      S^T (32 keys x 32 heads) = C (keys x D_qk) * Q^T on v_mfma_f32_32x32x16_bf16, Q^T held in
//           registers for the whole key loop, C read with ds_read_b128;
//   softmax fp32 online max/sum per head in base 2; the running max only moves when a tile exceeds it by
//           more than 2^8 (exact: numerator and denominator share the reference);
//   PV      O^T (D_v x 32 heads) += V^T (D_v x keys) * P^T. V^T comes from the same row-major tile through
//           ds_read_b64_tr_b16 (each 16-lane group reads a 4-key x 16-column block transposed); P^T is the
//           S^T accumulator itself, converted to bf16 (the product's K order is the accumulator's row
//           order, and the transposed reads fetch the keys in that order). O stays in AGPRs.
// Decode batches with few rows split the key list across workgroups; each split writes its own softmax output
// (bf16) with its (m, l), and a second pass merges them.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dsa {

template <int H, int DQK, int DV>
struct AttnCfg {
  static constexpr int NWAVE = H >= 128 ? 4 : (H + 31) / 32;   // waves per workgroup (32 heads each)
  static constexpr int HG = NWAVE * 32;                          // heads per workgroup
  static constexpr int NHG = (H + HG - 1) / HG;                  // head groups per row
  static constexpr int NT = NWAVE * kWave;
  static constexpr int KS = DQK / 16;             // K steps (16 wide) of the QK product
  static constexpr int MT = DV / 32;              // 32-row M tiles of the PV product
  static constexpr int BN = 32;                   // keys per tile
  static constexpr int ROWB = DQK * 2;            // bytes of one latent row
  static constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
  static constexpr bool SWZ = CPR % 8 == 0;       // chunk swizzle needs whole groups of 8 chunks
  static constexpr int TILE = BN * ROWB;          // bytes of one key tile
  static constexpr int NBUF = 4;                  // tiles t-1 (PV), t (QK), t+1 and t+2 (in flight)
  static constexpr int WLOADS = BN * CPR / kWave; // wave-wide 1 KB loads per tile
  static constexpr int PER = WLOADS / NWAVE;      // loads per wave per tile
  static constexpr int KMAX = 2048;               // longest key list of one workgroup (longer lists split)
  static constexpr int QL = KS >= 8 ? 1 : 0;      // trailing K steps of Q kept in LDS, not in registers
  static constexpr int QR = KS - QL;              // K steps of Q held in registers
  // the output rows go through LDS as whole 1 KB rows (each wave's 32 rows fit its share of the tile buffers)
  static constexpr bool OLDS = DV == 512 && H % 32 == 0 && NWAVE * 32 * 1024 <= NBUF * TILE;
  static_assert(DQK % 16 == 0 && DV % 32 == 0 && DV <= DQK, "attention tiling");
  static_assert(BN * CPR % kWave == 0 && WLOADS % NWAVE == 0, "every wave issues the same tile loads");
  static_assert(KMAX % NT == 0, "the prologue gives every thread the same number of list entries");
};

// Physical 16-byte chunk of logical chunk c in row `row` (an involution on the low 3 bits). gfx950's LDS
// serves 256 bytes (64 banks) per cycle: a ds_read_b128 phase is 16 lanes, a ds_read_b64_tr_b16 phase 32.
// Rows are 1152 bytes, so consecutive rows alternate between the two 128-byte halves of the bank space.
// With f(row) = 4*((row >> 1) & 1) + ((row >> 2) & 3):
//   - a QK read phase (16 consecutive rows, one chunk) hits 16 distinct 16-byte bank groups: within each
//     half, the 8 rows get 8 distinct f;
//   - a PV read phase (4 consecutive rows from a multiple of 4, 4 chunks from a multiple of 4) does too:
//     the two rows of a half differ in bit 2 of f, which moves the aligned 4-chunk group to the other one.
template <bool SWZ>
__device__ __forceinline__ int swz(int c, int row) {
  if constexpr (SWZ) return c ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  return c;
}

// The same load as a plain (non-volatile) asm statement: it does not fence the LDS reads around it, so the
// QK block can keep its reads running ahead across the gather. Its output register is never written; the
// caller folds it into a value that is consumed after the key loop, which keeps the statement alive and in
// its iteration. It must not move above the barrier that frees its buffer: its address comes from an LDS
// read issued after that barrier.
__device__ __forceinline__ uint32_t load_lds_16_free(uint64_t src, uint32_t lds_base) {
  uint32_t token;
  asm("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" : "=v"(token) : "v"(src), "s"(lds_base));
  return token;
}

// The same load with a 32-bit byte offset from a 64-bit base held in SGPRs (the saddr form): address = base + voff.
__device__ __forceinline__ uint32_t load_lds_16_off(uint32_t voff, uint64_t base, uint32_t lds_base) {
  uint32_t token;
  asm("s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" : "=v"(token) : "v"(voff), "s"(base), "s"(lds_base));
  return token;
}
__device__ __forceinline__ void load_lds_16_off_fenced(uint32_t voff, uint64_t base, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds_base)
               : "memory");
}

// S^T accumulation of the QK product in VGPRs (the builtin would put it in AGPRs, which O fills). The
// compiler's hazard tracking does not see inside inline asm, so the wait states it would insert are spelled
// out: two before a tile's first MFMA (a VALU write of an operand register just before it), and 20 after the
// last one (an 8-pass XDL result read by VALU; s_nop n gives n + 1). Back-to-back accumulation into the same
// registers needs none.
__device__ __forceinline__ void mfma_s_first(f32x16 &c, bf16x8 a, bf16x8 b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_next(f32x16 &c, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_last(f32x16 &c, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(c) : "v"(a), "v"(b));
}
// Register copy the optimiser cannot see through (not volatile: it may still move with its input).
__device__ __forceinline__ uint32_t opaque_u32(uint32_t v) {
  asm("" : "+v"(v));
  return v;
}

// Split workspace: bf16 partial outputs [num_q, splits, H, D_v], then fp32 (m, l) [num_q, splits, H, 2] at this
// float offset (D_v is even, so the partials end on a 4-byte boundary; rounded up to 16 bytes).
__host__ __device__ __forceinline__ size_t sparse_attn_ws_ml_offset(int num_q, int splits, int H, int D_v) {
  return ((size_t)num_q * splits * H * D_v / 2 + 3) / 4 * 4;
}

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;   // 32-bit LDS addresses

// OFF32: every selected row lies within 4 GB of the latent base, so the prologue keeps each row's byte offset
// (slot * row bytes, 0 for the padding past the list) and a gather load adds only its chunk offset to it.
template <int H, int DQK, int DV, bool OFF32>
__global__ __launch_bounds__((H >= 128 ? 4 : (H + 31) / 32) * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sparse_attn_kernel(AttnArgs a, int keys_per_split) {
  using C = AttnCfg<H, DQK, DV>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_tile[C::NBUF * C::TILE];
  __shared__ uint32_t lds_slot[C::KMAX];         // cache rows of the selected entries, compacted; ~0u = none
  __shared__ __attribute__((aligned(16))) u32x4 lds_q[C::QL > 0 ? C::NWAVE * C::QL * kWave : 1];
  __shared__ uint32_t lds_cnt[C::KMAX / C::NT * C::NWAVE];   // per-wave entry counts of each group

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps wave-derived offsets scalar
  const int n = lane & 31, g = lane >> 5;        // MFMA row/column index and half-wave
  // unit -> (row, head group, split): every unit of row r lands on XCD r % 8 (workgroups go round-robin
  // over the 8 XCDs), and the last rows (longest key lists in a prefill) are dispatched first
  const int u = blockIdx.x;
  const int row_blocks = (a.num_q + 7) / 8;
  const int inner = u / 8 / row_blocks;                           // split * NHG + head group
  const int r = a.num_q - 1 - ((u / 8) % row_blocks * 8 + u % 8);
  if (r < 0) return;
  const int hg = inner % C::NHG, split = inner / C::NHG;
  const int b = a.q_seq[r];
  const int p_r = a.q_pos[r];
  const int head = hg * C::HG + wv * 32 + n;
  const int i_lo = split * keys_per_split;
  const int nlist = max(0, min(a.k, i_lo + keys_per_split) - i_lo);
  const int32_t *idx_row = a.idx + (int64_t)r * a.k + i_lo;
  const uint8_t *latent = (const uint8_t *)a.latent;

  // ---- prologue: addresses of the rows to attend, compacted in list order (entries that are -1 or outside
  //      0..p_r are dropped here, so they cost nothing later; the softmax does not depend on the order).
  //      Each thread loads all of its list entries (at most KMAX / NT) up front, with the Q loads behind them,
  //      and the per-wave counts of every group go through LDS at once: the row pays one memory latency and
  //      two barriers here, not a latency and two barriers per NT entries.
  constexpr int PE = C::KMAX / C::NT;
  int ent[PE];
#pragma unroll
  for (int e = 0; e < PE; ++e) {
    const int i = e * C::NT + tid;
    ent[e] = i < nlist ? idx_row[i] : -1;
  }
  // Paged caches (never OFF32): every entry's page id is loaded once the list has landed and before the Q loads
  // go out (entries outside 0..p_r read the sequence's first page id, never used), so the slots wait for one
  // page-table latency and not for Q; contiguous caches load nothing more here.
  const bool paged = !OFF32 && a.slot.page_table != nullptr;
  int pid[PE];
  if (paged) {
    const int32_t *ptab = a.slot.page_table + (int64_t)b * a.slot.max_pages;
#pragma unroll
    for (int e = 0; e < PE; ++e) {
      const bool ok = ent[e] >= 0 && ent[e] <= p_r;
      pid[e] = ptab[ok ? ent[e] >> a.slot.page_shift : 0];
    }
  }
  // Q^T fragments of this wave's 32 heads (B operand: column = head, 8 consecutive d per half-wave). The K
  // steps kept in LDS wait in q_tail until tile 0 has landed, so no wait for Q comes before the first gather:
  // the Q loads and the first tiles' gathers are in flight together.
  bf16x8 qf[C::QR];
  u32x4 q_tail[C::QL > 0 ? C::QL : 1];
#pragma unroll
  for (int s = 0; s < C::KS; ++s) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (H % 32 == 0 || head < H)
      v = *(const u32x4 *)((const uint16_t *)a.q + ((int64_t)r * H + head) * DQK + s * 16 + g * 8);
    if (s < C::QR) qf[s < C::QR ? s : 0] = __builtin_bit_cast(bf16x8, v);
    else q_tail[s - C::QR] = v;
  }
  uint32_t sl[PE];
  if (paged) {
    const int mask = (1 << a.slot.page_shift) - 1;
#pragma unroll
    for (int e = 0; e < PE; ++e) {
      const bool ok = ent[e] >= 0 && ent[e] <= p_r;
      sl[e] = ok ? (uint32_t)(((int64_t)pid[e] << a.slot.page_shift) + (ent[e] & mask)) : 0u;
    }
  } else {
    const int64_t seq0 = (int64_t)b * a.slot.seq_stride;
#pragma unroll
    for (int e = 0; e < PE; ++e) {
      const bool ok = ent[e] >= 0 && ent[e] <= p_r;
      if constexpr (OFF32) sl[e] = ok ? (uint32_t)(seq0 + ent[e]) * (uint32_t)C::ROWB : 0u;
      else sl[e] = ok ? (uint32_t)(seq0 + ent[e]) : 0u;
    }
  }
  uint64_t msk[PE];
#pragma unroll
  for (int e = 0; e < PE; ++e) {
    const bool ok = ent[e] >= 0 && ent[e] <= p_r;
    msk[e] = ballot(ok);
    if (lane == 0) lds_cnt[e * C::NWAVE + wv] = (uint32_t)__popcll(msk[e]);
  }
  __syncthreads();
  int nkeys = 0;
#pragma unroll
  for (int e = 0; e < PE; ++e) {
    int before = nkeys, total = nkeys;
    for (int w = 0; w < C::NWAVE; ++w) {
      const int c = (int)lds_cnt[e * C::NWAVE + w];
      before += w < wv ? c : 0;
      total += c;
    }
    if ((msk[e] >> lane) & 1) lds_slot[before + lanes_below(msk[e])] = sl[e];
    nkeys = total;
  }
  __syncthreads();
  const int ntiles = (nkeys + C::BN - 1) / C::BN;
  for (int i = nkeys + tid; i < ntiles * C::BN; i += C::NT) lds_slot[i] = OFF32 ? 0u : ~0u;   // tail of the last tile
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds_tile;
  // this lane's part of every tile load (loop invariant): load j fills LDS slot P = (j * NWAVE + wv) * 64 + lane,
  // i.e. row P / CPR at its swizzled chunk; packed as (row << 16) | byte offset within the row
  uint32_t ld_pk[C::PER];
#pragma unroll
  for (int j = 0; j < C::PER; ++j) {
    const uint32_t P = (uint32_t)((j * C::NWAVE + wv) * kWave + lane);
    const uint32_t row = P / C::CPR, phys = P - row * C::CPR;
    ld_pk[j] = (row << 16) | (uint32_t)(16 * swz<C::SWZ>((int)phys, (int)row));
  }
  __syncthreads();

  // Gather of one tile, split in two: the row addresses (one LDS round trip), then the wave's PER loads, which
  // the QK block below spreads between its MFMAs. Missing rows load row 0 of the pool instead (finite data,
  // masked out of the softmax), so a wave always issues PER loads.
  // (ld_pk goes through an opaque copy each tile: values derived from it would otherwise be hoisted out of the
  // key loop and held in registers for its whole length)
  auto gather_rows = [&](int t, uint32_t (&rows)[C::PER], uint32_t (&pk)[C::PER]) {
#pragma unroll
    for (int j = 0; j < C::PER; ++j) pk[j] = (uint32_t)opaque((int)ld_pk[j]);
#pragma unroll
    for (int j = 0; j < C::PER; ++j) rows[j] = lds_slot[t * C::BN + (pk[j] >> 16)];
  };
  // In the key loop the loads may float within their iteration (load_lds_16_free); the two tiles loaded before
  // it must stay in issue order ahead of the first wait, so those use the fenced form.
  uint32_t sink = 0;   // see load_lds_16_free
  auto gather_load = [&](int t, const uint32_t (&rows)[C::PER], const uint32_t (&pk)[C::PER], int j,
                         bool fenced = false) {
    const uint32_t tile_lds = lds_base + (uint32_t)((t % C::NBUF) * C::TILE);
    const uint32_t dst = tile_lds + (uint32_t)((j * C::NWAVE + wv) * kWave * 16);
    if constexpr (OFF32) {
      const uint32_t voff = rows[j] + (pk[j] & 0xffffu);
      if (fenced) load_lds_16_off_fenced(voff, (uint64_t)latent, dst);
      else sink ^= load_lds_16_off(voff, (uint64_t)latent, dst);
    } else {
      const uint64_t keep = 0ull - (uint64_t)(rows[j] != ~0u);   // arithmetic select, no branch
      const uint64_t src = (uint64_t)latent + (((uint64_t)rows[j] * C::ROWB + (pk[j] & 0xffffu)) & keep);
      if (fenced) load_lds_16(src, dst);
      else sink ^= load_lds_16_free(src, dst);
    }
  };
  // K step s of the QK block issues gather load j when s == load_step(j): the first waits two MFMAs for its row
  // address, the rest are spread evenly over the block
  constexpr auto load_step = [](int j) { return 2 + j * (C::KS - 2) / C::PER; };

  // lane offsets of the QK reads: key row n, logical chunk 2s + g; the swizzle only touches the low 3 chunk
  // bits, so step s reads at base[s & 3] + 128 * (s >> 2)
  uint32_t qk_base[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) qk_base[v] = (uint32_t)(n * C::ROWB + 16 * swz<C::SWZ>(2 * v + g, n));
  // lane offsets of the transposed V reads: 16-lane group (g, dh) reads keys 16s + 8h + 4g + (i >> 2) and
  // columns 32*mt + 16*dh + 4*(i & 3) .. +3; their swizzle term depends on h (key bit 3) but not on s or mt,
  // so (M tile mt, half h) reads at base[h][mt & 1] + 128 * (mt >> 1) + 16s rows
  const int gi = lane & 15, dh = (lane >> 4) & 1;
  uint32_t tr_base[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int key = 8 * h + 4 * g + (gi >> 2);
      const int col = 32 * v + 16 * dh + 4 * (gi & 3);
      tr_base[h][v] = (uint32_t)(key * C::ROWB + 16 * swz<C::SWZ>(col >> 3, key) + (col & 7) * 2);
    }
  auto lds_ptr = [](uint32_t addr) { return (const lds_u8 *)(uintptr_t)addr; };

  // ---- S^T = C Q^T for tile t (keys x heads, this lane: head n, keys (i/4)*8 + 4g + i%4), gathering tile t + 2
  //      on the way when `gather` is set
  auto qk = [&](int t, auto gather_tag, f32x16 &S) {
    constexpr bool gather = decltype(gather_tag)::value;
    const uint32_t tb = lds_base + (uint32_t)((t % C::NBUF) * C::TILE);
    uint32_t rows[C::PER], pk[C::PER];
    if constexpr (gather) gather_rows(t + 2, rows, pk);
    uint32_t qb[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) qb[v] = opaque_u32(tb + (C::SWZ ? qk_base[v] : 0u));
    auto rd = [&](int s) {
      const uint32_t addr = C::SWZ ? qb[s & 3] + 128u * (uint32_t)(s >> 2)
                                   : tb + (uint32_t)(n * C::ROWB + 16 * (2 * s + g));
      return __builtin_bit_cast(bf16x8, *(const __attribute__((address_space(3))) u32x4 *)lds_ptr(addr));
    };
    constexpr int LA = 3;   // LDS reads in flight ahead of the MFMA that consumes them
    bf16x8 kf[LA + 1];
#pragma unroll
    for (int s = 0; s < LA && s < C::KS; ++s) kf[s] = rd(s);
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      if (s + LA < C::KS) kf[(s + LA) % (LA + 1)] = rd(s + LA);
      const bf16x8 bq = s < C::QR ? qf[s < C::QR ? s : 0]
                                  : __builtin_bit_cast(bf16x8, lds_q[(wv * C::QL + (s - C::QR)) * kWave + lane]);
      if (s == 0) mfma_s_first(S, kf[0], bq);
      else if (s == C::KS - 1) mfma_s_last(S, kf[s % (LA + 1)], bq);
      else mfma_s_next(S, kf[s % (LA + 1)], bq);
      if constexpr (gather) {
#pragma unroll
        for (int j = 0; j < C::PER; ++j)
          if (load_step(j) == s) gather_load(t + 2, rows, pk, j);
      }
      __builtin_amdgcn_sched_barrier(0);   // keep each step's read LA steps ahead of its MFMA
    }
    if constexpr (gather) {
#pragma unroll
      for (int j = 0; j < C::PER; ++j)
        if (load_step(j) >= C::KS) gather_load(t + 2, rows, pk, j);
    }
  };

  // ---- online softmax of tile t in base 2, scores kept unscaled: m_run is the running max of
  //      scale2 * score; it only moves when a tile exceeds it by more than 2^8 (exact: numerator and
  //      denominator share the reference). Produces the bf16 P^T operands and the tile's row-sum part.
  const float scale2 = a.sm_scale * 1.4426950408889634f;  // > 0 (checked by the host)
  float m_run = -INFINITY, l_run = 0.f;
  auto softmax = [&](int t, f32x16 &S, bf16x8 (&pf)[2], float &alpha) -> bool {
    const int nv = nkeys - t * C::BN;   // valid keys of this tile (compacted list: a prefix)
    if (nv < C::BN) {   // last tile only
      const int g4 = opaque(4 * g);   // keeps the 16 key numbers from being hoisted out of the loop
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((i >> 2) * 8 + g4 + (i & 3) >= nv) S[i] = -INFINITY;
    }
    float tmax = S[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, S[i]);
    tmax = xor32_max(tmax) * scale2;
    const bool move = tmax > m_run + 8.f;
    const float m_new = move ? tmax : m_run;
    alpha = move ? exp2f(m_run - m_new) : 1.f;  // m_run = -inf gives 0 (O and l are 0 then)
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      S[i] = __builtin_amdgcn_exp2f(fmaf(S[i], scale2, -m_new));  // v_exp_f32; -inf gives 0
      lsum += S[i];
    }
    l_run = l_run * alpha + lsum;
    // P^T operand of K step s: this lane's accumulator registers 8s .. 8s+7 (keys 16s + 8(j/4) + 4g + j%4)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4 v = {pack_bf16x2(S[8 * s + 0], S[8 * s + 1]), pack_bf16x2(S[8 * s + 2], S[8 * s + 3]),
                       pack_bf16x2(S[8 * s + 4], S[8 * s + 5]), pack_bf16x2(S[8 * s + 6], S[8 * s + 7])};
      pf[s] = __builtin_bit_cast(bf16x8, v);
    }
    return move;
  };

  f32x16 o[C::MT];
#pragma unroll
  for (int t = 0; t < C::MT; ++t) o[t] = f32x16{};

  // ---- O^T += V^T P^T for tile t, V^T read transposed from the row-major tile
  auto pv = [&](int t, const bf16x8 (&pf)[2]) {
    const uint32_t tb = lds_base + (uint32_t)((t % C::NBUF) * C::TILE);
    uint32_t trp[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int v = 0; v < 2; ++v) trp[h][v] = opaque_u32(tb + (C::SWZ ? tr_base[h][v] : 0u));
    auto rd = [&](int i) {   // A operand of step i = 16 s + mt
      const int s = i / C::MT, mt = i % C::MT;
      u32x2 half[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t addr;
        if constexpr (C::SWZ) {
          addr = trp[h][mt & 1] + 128u * (uint32_t)(mt >> 1) + (uint32_t)(16 * s * C::ROWB);
        } else {
          const int key = 16 * s + 8 * h + 4 * g + (gi >> 2), col = 32 * mt + 16 * dh + 4 * (gi & 3);
          addr = tb + (uint32_t)(key * C::ROWB + 2 * col);
        }
        half[h] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v *)lds_ptr(addr)));
      }
      return __builtin_bit_cast(bf16x8, u32x4{half[0].x, half[0].y, half[1].x, half[1].y});
    };
    constexpr int NS = 2 * C::MT, LA = 2;
    bf16x8 vf[LA + 1];
#pragma unroll
    for (int i = 0; i < LA && i < NS; ++i) vf[i] = rd(i);
#pragma unroll
    for (int i = 0; i < NS; ++i) {   // consecutive MFMAs update different accumulators
      if (i + LA < NS) vf[(i + LA) % (LA + 1)] = rd(i + LA);
      o[i % C::MT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % (LA + 1)], pf[i / C::MT], o[i % C::MT], 0, 0, 0);
    }
  };
  // O *= alpha per head, in AGPRs (VALU cannot read AGPRs directly). The first wait covers the last PV MFMA's
  // AGPR writes (hidden from the compiler by the asm), the last one the next PV MFMA reading them.
  auto rescale = [&](float alpha) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
    for (int t2 = 0; t2 < C::MT; ++t2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float tmp;
        asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                     : "+a"(o[t2][i]), "=&v"(tmp) : "v"(alpha));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_nop 4" ::: "memory");
  };

  // Software pipeline over the tiles: iteration t runs QK(t) (gathering tile t + 2 meanwhile), then the
  // softmax of tile t interleaved with PV(t - 1). Four tile buffers: t - 1, t, and t + 1, t + 2 in flight.
  f32x16 S;
  bf16x8 pf_prev[2], pf_cur[2];
  if (ntiles > 0) {
    uint32_t rows[C::PER], pk[C::PER];
    gather_rows(0, rows, pk);
#pragma unroll
    for (int j = 0; j < C::PER; ++j) gather_load(0, rows, pk, j, true);
    if (ntiles > 1) {
      gather_rows(1, rows, pk);
#pragma unroll
      for (int j = 0; j < C::PER; ++j) gather_load(1, rows, pk, j, true);
    }
    // tile 0 (the Q loads, issued before the gathers, have landed too: loads complete in order)
    if (ntiles > 1) wait_vmcnt<C::PER>(); else wait_vmcnt<0>();
#pragma unroll
    for (int s = 0; s < C::QL; ++s) lds_q[(wv * C::QL + s) * kWave + lane] = q_tail[s];   // this wave's own part
    lds_barrier();
    if (ntiles > 2) qk(0, std::true_type{}, S); else qk(0, std::false_type{}, S);
    float alpha;
    softmax(0, S, pf_prev, alpha);   // O is still 0: nothing to rescale
  } else {
    // no tile: wait for the Q loads anyway, so that no path reaches the key loop with them outstanding (the
    // compiler would otherwise wait for them inside the loop, draining the tile loads each time)
    wait_vmcnt<0>();
  }
  for (int t = 1; t < ntiles; ++t) {
    // tile t has landed once at most the next tile's loads are outstanding (loads complete in order)
    if (t + 1 < ntiles) wait_vmcnt<C::PER>(); else wait_vmcnt<0>();
    lds_barrier();  // tile t visible to every wave; every wave is done with tiles t - 2 (PV) and t - 1 (QK)
    if (t + 2 < ntiles) qk(t, std::true_type{}, S); else qk(t, std::false_type{}, S);
    float alpha;
    const bool move = softmax(t, S, pf_cur, alpha);
    pv(t - 1, pf_prev);
    // The probabilities of tile t are needed here, before the branch: otherwise the compiler sinks their
    // exponentials past it, out of the block where they overlap the PV MFMAs.
    asm volatile("" ::"v"(pf_cur[0]), "v"(pf_cur[1]), "v"(l_run));
    if (ballot(move)) rescale(alpha);   // O must hold the tiles before t, relative to the old max
    pf_prev[0] = pf_cur[0];
    pf_prev[1] = pf_cur[1];
  }
  if (ntiles > 0) pv(ntiles - 1, pf_prev);
  asm volatile("" ::"v"(sink));

  const float l_tot = xor32_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // destination of this wave's 32 heads: rows of DV values, head after head (the output, or this split's
  // partial: its own softmax output O / l as bf16, merged by attn_combine_kernel; the merge weights are convex,
  // so this adds at most the bf16 rounding the final output has anyway)
  uint16_t *dst = a.splits == 1 ? (uint16_t *)a.out + ((int64_t)r * H + hg * C::HG + wv * 32) * DV
                                : (uint16_t *)a.ws + (((int64_t)r * a.splits + split) * H + hg * C::HG + wv * 32) * DV;
  if constexpr (C::OLDS) {
    // Through LDS, so that every store writes one head's whole 1 KB row: the wave's 32 rows form one
    // contiguous 32 KB block (written straight from the accumulator layout, each lane's 8-byte pieces land
    // in 32 rows 1 KB apart). Rows sit in this wave's 32 KB of the tile buffers, free once every wave has
    // finished its last PV; 16-byte chunk c of row h is stored at chunk c ^ (h & 15), so the row reads are
    // conflict-free and the writes two-way.
    __syncthreads();
    const uint32_t obase = lds_base + (uint32_t)wv * 32u * 1024u;
#pragma unroll
    for (int t = 0; t < C::MT; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x2 v = {pack_bf16x2(o[t][q4 * 4 + 0] * inv, o[t][q4 * 4 + 1] * inv),
                         pack_bf16x2(o[t][q4 * 4 + 2] * inv, o[t][q4 * 4 + 3] * inv)};
        const uint32_t c = (uint32_t)(t * 4 + q4) ^ (uint32_t)(n & 15);
        *(__attribute__((address_space(3))) u32x2 *)(uintptr_t)(obase + (uint32_t)n * 1024u + c * 16u + (uint32_t)g * 8u) =
            v;
      }
#pragma unroll 8
    for (int h = 0; h < 32; ++h) {
      const uint32_t c = (uint32_t)lane ^ (uint32_t)(h & 15);
      const u32x4 v = *(const __attribute__((address_space(3))) u32x4 *)(uintptr_t)(obase + (uint32_t)h * 1024u + c * 16u);
      *(u32x4 *)(dst + h * DV + lane * 8) = v;
    }
  } else {
    if (H % 32 == 0 || head < H) {
#pragma unroll
      for (int t = 0; t < C::MT; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(u32x2 *)(dst + n * DV + t * 32 + q4 * 8 + g * 4) =
              u32x2{pack_bf16x2(o[t][q4 * 4 + 0] * inv, o[t][q4 * 4 + 1] * inv),
                    pack_bf16x2(o[t][q4 * 4 + 2] * inv, o[t][q4 * 4 + 3] * inv)};
    }
  }
  if (H % 32 != 0 && head >= H) return;
  if (a.splits == 1) {
    if (a.lse != nullptr && g == 0)
      a.lse[(int64_t)r * H + head] = l_tot > 0.f ? m_run * 0.6931471805599453f + logf(l_tot) : -INFINITY;
  } else if (g == 0) {
    float *ml = a.ws + sparse_attn_ws_ml_offset(a.num_q, a.splits, H, DV) + (((int64_t)r * a.splits + split) * H + head) * 2;
    ml[0] = m_run;
    ml[1] = l_tot;
  }
}

// Merge of the split partials: out = sum_j w_j Obar_j with w_j = 2^(m_j - M) l_j / L, L = sum_j 2^(m_j - M) l_j,
// M = max_j m_j over the splits that saw a key (l_j > 0), Obar_j the split's own softmax output (bf16). One
// workgroup = one row x HPW heads; a thread owns 16 consecutive outputs of one head. Splits are taken SB at a
// time and every load of a batch goes out before any is used (indexes past the last split repeat it and are
// weighted 0), so up to SB splits cost one memory latency: (m, l) and the partial rows together when the row
// has at most SB splits, else one pass over (m, l) for M and one over the batches. The launch picks the
// smallest SB of 2, 4, 8 that holds the row's splits, so no load repeats another when they fit one batch.
template <int DV, int SB>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int TPH = DV / 16;          // threads per head
  constexpr int HPW = 256 / TPH;        // heads per workgroup
  static_assert(DV % 16 == 0 && 256 % TPH == 0, "combine tiling");
  const int groups = (a.H + HPW - 1) / HPW;
  const int r = blockIdx.x / groups;
  const int h = (blockIdx.x - r * groups) * HPW + (int)threadIdx.x / TPH;
  const int d0 = ((int)threadIdx.x % TPH) * 16;
  if (h >= a.H) return;
  const int S = a.splits;
  const float *ml = a.ws + sparse_attn_ws_ml_offset(a.num_q, S, a.H, DV);   // [num_q, splits, H, 2]: (m, l)
  const f32x2 *mlh = (const f32x2 *)ml + (int64_t)r * S * a.H + h;          // split j at mlh[j * H]
  const u32x4 *poh = (const u32x4 *)((const uint16_t *)a.ws + ((int64_t)r * S * a.H + h) * DV + d0);
  const int64_t pstride = (int64_t)a.H * DV / 8;                            // u32x4 per split
  float M = -INFINITY;
  if (S > SB) {
    for (int j0 = 0; j0 < S; j0 += SB) {
      f32x2 v[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u) v[u] = mlh[(int64_t)min(j0 + u, S - 1) * a.H];
#pragma unroll
      for (int u = 0; u < SB; ++u)
        if (j0 + u < S && v[u].y > 0.f) M = fmaxf(M, v[u].x);
    }
  }
  float L = 0.f;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  for (int j0 = 0; j0 < S; j0 += SB) {
    f32x2 v[SB];
    u32x4 w[SB][2];
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int j = min(j0 + u, S - 1);
      v[u] = mlh[(int64_t)j * a.H];
      w[u][0] = poh[j * pstride];
      w[u][1] = poh[j * pstride + 1];
    }
    if (S <= SB) {
#pragma unroll
      for (int u = 0; u < SB; ++u)
        if (u < S && v[u].y > 0.f) M = fmaxf(M, v[u].x);
    }
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const float f = j0 + u < S && v[u].y > 0.f ? exp2f(v[u].x - M) * v[u].y : 0.f;   // an empty split weighs 0
      L += f;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t ww[4] = {w[u][q].x, w[u][q].y, w[u][q].z, w[u][q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[q * 8 + 2 * e] = fmaf(f, bf16_lo(ww[e]), acc[q * 8 + 2 * e]);
          acc[q * 8 + 2 * e + 1] = fmaf(f, bf16_hi(ww[e]), acc[q * 8 + 2 * e + 1]);
        }
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t *orow = (uint16_t *)a.out + ((int64_t)r * a.H + h) * DV + d0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const u32x4 w = {pack_bf16x2(acc[q * 8 + 0] * inv, acc[q * 8 + 1] * inv),
                     pack_bf16x2(acc[q * 8 + 2] * inv, acc[q * 8 + 3] * inv),
                     pack_bf16x2(acc[q * 8 + 4] * inv, acc[q * 8 + 5] * inv),
                     pack_bf16x2(acc[q * 8 + 6] * inv, acc[q * 8 + 7] * inv)};
    *(u32x4 *)(orow + 8 * q) = w;
  }
  if (d0 == 0 && a.lse != nullptr)
    a.lse[(int64_t)r * a.H + h] = L > 0.f ? M * 0.6931471805599453f + logf(L) : -INFINITY;
}

size_t sparse_attn_ws_floats(int num_q, int splits, int H, int D_v) {
  if (splits <= 1) return 0;
  return sparse_attn_ws_ml_offset(num_q, splits, H, D_v) + (size_t)num_q * splits * H * 2;
}

template <int H, int DQK, int DV>
static hipError_t launch_t(const AttnArgs &a, hipStream_t st) {
  using C = AttnCfg<H, DQK, DV>;
  int kps = (a.k + a.splits - 1) / a.splits;
  kps = (kps + C::BN - 1) / C::BN * C::BN;
  if (kps > C::KMAX) return hipErrorInvalidValue;   // the caller plans enough splits
  const int units = (a.num_q + 7) / 8 * 8 * C::NHG * a.splits;
  // 32-bit row offsets when every slot the batch can address lies within 4 GB of the base: contiguous caches
  // with (num_seqs - 1) * seq_stride + max_kv_len rows (the host knows it); paged caches keep 64-bit addresses
  if (a.max_slots > 0 && a.max_slots * (int64_t)C::ROWB <= (int64_t)0xFFFFFFFFll - C::ROWB)
    hipLaunchKernelGGL((sparse_attn_kernel<H, DQK, DV, true>), dim3(units), dim3(C::NT), 0, st, a, kps);
  else
    hipLaunchKernelGGL((sparse_attn_kernel<H, DQK, DV, false>), dim3(units), dim3(C::NT), 0, st, a, kps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  constexpr int HPW = 256 / (DV / 16);
  const dim3 grid(a.num_q * ((a.H + HPW - 1) / HPW));
  if (a.splits <= 2)
    hipLaunchKernelGGL((attn_combine_kernel<DV, 2>), grid, dim3(256), 0, st, a);
  else if (a.splits <= 4)
    hipLaunchKernelGGL((attn_combine_kernel<DV, 4>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_combine_kernel<DV, 8>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const AttnArgs &a, hipStream_t st) {
  if (a.H == 128 && a.D_qk == 576 && a.D_v == 512) return launch_t<128, 576, 512>(a, st);
  if (a.H == 8 && a.D_qk == 80 && a.D_v == 64) return launch_t<8, 80, 64>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace dsa

// Device-side helpers shared by the libdsa kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Physical cache row of logical position s of sequence b (contiguous or paged layout).
struct SlotMap {
  const int32_t *page_table;  // [num_seqs * max_pages] or nullptr
  int64_t seq_stride;
  int32_t max_pages;
  int32_t page_shift;         // log2(page_size) when paged
  __device__ __forceinline__ int64_t operator()(int b, int s) const {
    if (page_table == nullptr) return (int64_t)b * seq_stride + s;
    const int page = page_table[(int64_t)b * max_pages + (s >> page_shift)];
    return ((int64_t)page << page_shift) + (s & ((1 << page_shift) - 1));
  }
};

// 16-byte load from global memory through a pointer the compiler cannot prove global (e.g. read from LDS).
__device__ __forceinline__ u32x4 load_global_16(const void *p) {
  return *(const __attribute__((address_space(1))) u32x4 *)(p);
}

// An opaque copy of v: stops the compiler from hoisting address arithmetic derived from v out of a loop
// (hoisted 64-bit addresses would otherwise stay live across the loop and spill).
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Wait until at most N vector memory operations of this wave are outstanding (loads and stores alike).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16-byte global -> LDS load of one wave: lane i's 16 bytes land at LDS byte address m0 + 16 * i. Issued as
// inline asm so that the compiler, which cannot see which tile a later LDS read touches, does not drain every
// load in flight before each read; completion is waited for explicitly (wait_vmcnt) before the tile is used.
__device__ __forceinline__ void load_lds_16(uint64_t src, uint32_t lds_base) {
  // s_nop: one wait state between writing M0 and the load that reads it
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base) : "memory");
}

// 16-byte buffer -> LDS load of one wave: lane i's 16 bytes come from rsrc.base + voff + OFF and land at LDS byte
// address m0 + OFF + 16 * i. Bytes at or past the resource's num_records read as zero. Inline asm for the same
// reason as load_lds_16.
template <int OFF>
__device__ __forceinline__ void load_lds_16_buf(u32x4 rsrc, uint32_t voff, uint32_t m0) {
  static_assert(OFF >= 0 && OFF < 4096, "MUBUF immediate offset");
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen offset:%3 lds" ::"v"(voff),
               "s"(rsrc), "s"(m0), "i"(OFF)
               : "memory");
}

// Raw buffer resource (stride 0) over [base, base + bytes): accesses at or past `bytes` are dropped (stores) or
// read zero (loads). base and bytes must be wave-uniform.
__device__ __forceinline__ u32x4 raw_rsrc(const void *base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  u32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)p);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu);
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = 0x00020000u;   // 32-bit data format, as untyped buffer accesses expect
  return r;
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations, then s_barrier. Unlike
// __syncthreads() it has no release fence, so outstanding global->LDS loads are NOT drained (their completion
// is waited for explicitly with s_waitcnt vmcnt). The memory clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

// Number of set bits of the wave mask below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Exact widening of bf16 bit patterns: the pattern is the high half of an fp32 word.
__device__ __forceinline__ float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 of two values, packed low|high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  // one v_cvt_pk_bf16_f32 (round to nearest even), lo in bits 0..15
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Four OCP E4M3 bytes -> four bf16 (exact: every E4M3 value is a bf16 value), packed as two dwords: gfx950's
// scaled packed convert, two bytes per instruction, with a scale of exactly 1.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t four) {
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(four, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(four, 1.0f, true));
  return r;
}

// Value of lane l ^ 32 (the other half-wave), via gfx950's v_permlane32_swap, which swaps lanes 32..63 of its first
// operand with lanes 0..31 of its second: with both operands equal it leaves (own, partner) in lanes 0..31 and
// (partner, own) in lanes 32..63, so the sum and the max below are the same in both halves.
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Wave-wide scans and reductions on DPP (VALU lane moves, no LDS round trip per step): row_shr 1, 2, 4, 8 build
// the prefix within each 16-lane row; row_bcast:15 then adds row 0's (row 2's) total to row 1 (row 3), and
// row_bcast:31 adds lanes 0..31's total to lanes 32..63. Lanes that a step does not write, or whose source lies
// outside their row, take `id` (the operation's identity), so the same steps serve add, min and max.
template <class Op>
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v, uint32_t id, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x111, 0xf, 0xf, false));   // row_shr:1
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x112, 0xf, 0xf, false));   // row_shr:2
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x114, 0xf, 0xf, false));   // row_shr:4
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x118, 0xf, 0xf, false));   // row_shr:8
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x142, 0xa, 0xf, false));   // row_bcast:15
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x143, 0xc, 0xf, false));   // row_bcast:31
  return v;
}
struct DppAdd {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};
struct DppMin {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; }
};
struct DppMax {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};
// Inclusive prefix sum over the wave, in lane order.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) { return wave_incl_scan_dpp(v, 0u, DppAdd{}); }
// Wave totals, the same in every lane (lane 63 holds the scan's total).
__device__ __forceinline__ uint32_t wave_total_sum(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan_dpp(v, 0u, DppAdd{}), 63);
}
__device__ __forceinline__ uint32_t wave_total_min(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan_dpp(v, 0xffffffffu, DppMin{}), 63);
}
__device__ __forceinline__ uint32_t wave_total_max(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan_dpp(v, 0u, DppMax{}), 63);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace dsa

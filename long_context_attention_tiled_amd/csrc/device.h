// Shared device-side types and helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace lcat {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Compile-time integer tag (selects a specialisation of a generic lambda).
template <int N>
struct Int {
  static constexpr int value = N;
};

// f(Int<0>{}), f(Int<1>{}), ..., f(Int<N-1>{}): a loop whose index is a
// constant expression in every step, independent of unrolling heuristics.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(Int<I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
constexpr float kLn2 = 0.6931471805599453f;

// 32x32 output tile, K = 16 per instruction.  Operand lane layout (wave64):
//   A: lane l holds A[l%32][8*(l/32) .. 8*(l/32)+7]
//   B: lane l holds B[8*(l/32) .. +7][l%32]
//   C: lane l, register r holds C[8*(r/4) + 4*(l/32) + r%4][l%32]
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16 output tile, K = 32 per instruction.
//   A: lane l holds A[l%16][8*(l/16) .. +7]
//   B: lane l holds B[8*(l/16) .. +7][l%16]
//   C: lane l, register r holds C[4*(l/16) + r][l%16]
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 ld_global_16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
// The same load with the non-temporal hint (nt bit).  Data read once and
// never again streams from HBM measurably faster this way on this part: a
// plain streaming read of a 4 GiB buffer reaches 6.1-6.3 TB/s, the same read
// with nt loads 6.8-7.1 TB/s.
__device__ __forceinline__ u32x4 ld_global_16_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ void st_global_16(void *p, u32x4 v) {
  *reinterpret_cast<u32x4 *>(p) = v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// fp32 -> bf16 with round-to-nearest-even (gfx950 converts in hardware).
__device__ __forceinline__ bf16 to_bf16(float x) { return static_cast<bf16>(x); }

__device__ __forceinline__ float bf16_to_f32(uint16_t bits) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(bits) << 16);
}

__device__ __forceinline__ float wave_shfl_xor(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Returns v unchanged but hides its value from the optimiser, so address
// arithmetic derived from it is recomputed where it is used (1-2 VALU ops)
// instead of being hoisted out of a loop and kept in registers.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Raw buffer descriptor over `bytes` bytes at `base` (gfx9-family word 3).
// Reads outside [0, bytes) return zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// 16-byte buffer load at voffset (per lane) + soffset (wave-uniform) bytes.
__device__ __forceinline__ u32x4 buf_load_16(__amdgpu_buffer_rsrc_t r, int voffset, int soffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, 0));
}
// The same with the non-temporal hint (cache-policy bit nt; see ld_global_16_nt).
__device__ __forceinline__ u32x4 buf_load_16_nt(__amdgpu_buffer_rsrc_t r, int voffset, int soffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, 2));
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor as four words (for inline assembly operands).
__device__ __forceinline__ u32x4 rsrc_words(const void *base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, (uint32_t)bytes, 0x00020000u};
}

// Global -> LDS copy without registers: lane l's 16 bytes at buffer offset
// `voffset` land at LDS address `lds_dst + 16 * l` (lds_dst wave-uniform).
// Lanes whose range check fails write zeros.  Completion is tracked by the
// wave's vector-memory counter only: a reader must wait_vmcnt() and then
// pass a barrier before using the data.  Issued from inline assembly so
// that the compiler does not also make every later LDS read wait for it.
// The statement declares no memory effects: it stays ordered with the other
// volatile statements (the barrier, the counter waits), and callers only
// target LDS that no wave reads before the next barrier.
__device__ __forceinline__ void dma_to_lds_16(u32x4 rsrc, char *lds_dst, int voffset) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void *)lds_dst;
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %2, 0 offen lds"
      :
      : "v"(voffset), "s"(m0), "s"(rsrc)
      : "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that neither waits for outstanding memory operations nor
// lets the compiler move memory operations across it.  LDS written by the
// DMA above is published by wait_vmcnt() + this barrier; LDS reads may stay
// in flight across it.
__device__ __forceinline__ void barrier_no_wait() { asm volatile("s_barrier" ::: "memory"); }

// Transposing LDS read (16-bit elements).  Within each group of 16 lanes,
// lane i receives element (i % 4) of the 8-byte rows addressed by lanes
// i/4, 4 + i/4, 8 + i/4 and 12 + i/4, in that order.
__device__ __forceinline__ u32x2 lds_read_tr16(const char *p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (__attribute__((address_space(3))) i16x4 *)p));
}

// max / sum of x over the lane pair (l, l ^ 32).
__device__ __forceinline__ float pair_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// max(a, b, c) / max(a, b) as single instructions.  fmaxf() first quiets
// possible signalling NaNs in its inputs (one extra instruction per input
// that comes straight from an MFMA); these skip that step and are meant for
// finite scores.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
__device__ __forceinline__ float max_raw(float a, float b) {
  float d;
  asm("v_max_f32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}
// max of x over the lane pair (l, l ^ 32), inputs assumed finite.
__device__ __forceinline__ float pair_max32_raw(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return max_raw(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

// Order of causal prefill work over the XCDs.  The dispatcher deals
// workgroups to the 8 XCDs in turn, so workgroup b runs on XCD b % 8 as the
// (b / 8)-th workgroup there, and each XCD has its own L2.  Work items are
// ranked by query block, longest rows first, times `per_q` combinations
// (batch, KV head, head slice): item = rank * per_q + combination.  The
// plain order (item = b) spreads the ranks an XCD runs at one time over
// 4 * 32 consecutive ranks (per_q = 2).  This order, when per_q divides 8,
// still keeps one combination per XCD, so that XCD streams one KV head
// through its L2, and hands the 8 / per_q XCDs of a combination their ranks
// in generations of kXcdCus consecutive ranks (one per CU), the XCDs taking
// the blocks of a generation in alternating directions so that their totals
// balance.  The workgroups an XCD runs together then walk nearly the same
// key prefix at the same time.  The result is a bijection of
// [0, n_qblk * per_q) whatever the part's layout; ranks past the last whole
// generation keep the plain order.
__device__ __forceinline__ int xcd_item(int b, int per_q, int n_qblk) {
  constexpr int kXcds = 8, kXcdCus = 32;
  if (per_q <= 0 || kXcds % per_q != 0) return b;
  const int m = kXcds / per_q;   // XCDs that share one combination
  const int x = b % kXcds, i = b / kXcds;
  const int gen = i / kXcdCus;
  if (gen >= n_qblk / (kXcdCus * m)) return b;
  const int xp = x / per_q, comb = x % per_q;
  const int blk = (gen & 1) ? m - 1 - xp : xp;
  return (kXcdCus * (m * gen + blk) + i % kXcdCus) * per_q + comb;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// acc + a.x + a.y for a pair of bf16 packed in one register (fp32 accumulate).
__device__ __forceinline__ float add_bf16_pair(uint32_t a, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), one, acc, false);
}

}  // namespace lcat

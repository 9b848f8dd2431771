// Shared device-side types and helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

}  // namespace lcat

// Pieces shared by the two FP8 prefill kernels (scores on FP8, and scores
// plus P V on FP8): the scaled FP8 MFMA, the 4-byte LDS DMA and the in-kernel
// quantisation of a wave's query rows.
//
// Operand layout of the scaled FP8 MFMA v_mfma_scale_f32_32x32x64_f8f6f4
// (measured on the part): for row r of A (or column r of B), lane r + 32h
// holds 32 bytes; bytes 0..15 of lanes r and r+32 form the first 32-element
// K block (K index 16h .. 16h+15 in lane r + 32h) and bytes 16..31 the
// second (K index 32 + 16h ..); the scale of block b comes from lane r + 32b,
// and op_sel k picks byte k of the scale register.  The 32x32 result has the
// usual layout: lane j + 32h, register i holds C[8 (i / 4) + 4h + i % 4][j].
#pragma once

#include "device.h"
#include "fp8_block.h"
#include "hadamard.h"

namespace lcat {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kE8m0One = 127;                 // E8M0 byte of 2^0
constexpr int kE8m0OneX4 = 0x7F7F7F7F;        // the same in every byte

// C + A B with the A block scales taken from byte SA of sa and the B block
// scales from byte SB of sb (both operands e4m3).
template <int SA, int SB>
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SA, sa, SB, sb);
}

// 4-byte global -> LDS copy per lane (lane l writes lds_dst + 4 l); the
// ordering rules are those of dma_to_lds_16.
__device__ __forceinline__ void dma_to_lds_4(u32x4 rsrc, char *lds_dst, int voffset) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void *)lds_dst;
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %0, %2, 0 offen lds"
      :
      : "v"(voffset), "s"(m0), "s"(rsrc)
      : "m0");
}

// A lane's 64 values of one query row as the two B operands of S^T = K Q^T
// on the scaled FP8 MFMA, for the lane in half gq of the wave: y[c][pt][e] is
// dim 64c + 32pt + 16gq + e, already multiplied by the query multiplier.
// Each block of 32 dims is quantised with the rule of fp8_block.h (the other
// 16 dims of a block sit in lane l ^ 32).  qf[c] covers dims 64c .. 64c+63:
// bytes 0..15 hold dims 64c + 16 gq .. +15 and bytes 16..31 dims
// 64c + 32 + 16 gq .. +15.  The returned scale word holds the E8M0 scale of
// block 2c + gq in byte 2c.
__device__ __forceinline__ int quantize_query_values(const float (&y)[2][2][16], int gq,
                                                     i32x8 (&qf)[2]) {
  int eb[2][2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      float am = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) am = fmaxf(am, fabsf(y[c][pt][e]));
      eb[c][pt] = fp8_block_exponent(pair_max32(am));
    }
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int e = -eb[c][pt];
        qf[c][4 * pt + w] = (int)fp8x4_rne(
            __builtin_amdgcn_ldexpf(y[c][pt][4 * w], e), __builtin_amdgcn_ldexpf(y[c][pt][4 * w + 1], e),
            __builtin_amdgcn_ldexpf(y[c][pt][4 * w + 2], e), __builtin_amdgcn_ldexpf(y[c][pt][4 * w + 3], e));
      }
  const int e0 = gq ? eb[0][1] : eb[0][0], e1 = gq ? eb[1][1] : eb[1][0];
  return (e0 + 127) | ((e1 + 127) << 16);
}

// One query row of head_dim 128 (qp: its first element): every element is
// multiplied by c2 in fp32, then quantised as above.
__device__ __forceinline__ int quantize_query_row(const bf16 *qp, int gq, float c2, i32x8 (&qf)[2]) {
  bf16x8 raw[2][2][2];   // [c][part][8 dims]
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        raw[c][pt][i] = as_bf16x8(ld_global_16(qp + 64 * c + 32 * pt + 16 * gq + 8 * i));
  float y[2][2][16];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int e = 0; e < 16; ++e) y[c][pt][e] = (float)raw[c][pt][e >> 3][e & 7] * c2;
  return quantize_query_values(y, gq, qf);
}

// The same row rotated first (hadamard.h): both lanes of a row take the
// whole row through the transform, each keeps its 64 dims, multiplies them
// by c2r (the query multiplier divided by 128) in fp32 and quantises them.
__device__ __forceinline__ int quantize_query_row_rotated(const bf16 *qp, int gq, float c2r,
                                                          const HadamardSigns &sg, i32x8 (&qf)[2]) {
  float v[128];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bf16x8 raw = as_bf16x8(ld_global_16(qp + 8 * i));
#pragma unroll
    for (int e = 0; e < 8; ++e) v[8 * i + e] = (float)raw[e];
  }
  hadamard128(v, sg);
  float y[2][2][16];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        y[c][pt][e] = (gq ? v[64 * c + 32 * pt + 16 + e] : v[64 * c + 32 * pt + e]) * c2r;
  return quantize_query_values(y, gq, qf);
}

}  // namespace lcat

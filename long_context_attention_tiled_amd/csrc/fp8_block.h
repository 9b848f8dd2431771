// Power-of-two block scales for FP8 (OCP e4m3) operands: the FP8 path of
// FA3 ("Flash Attention and distributed inference", §18.5) quantises blocks
// of the attention inputs.  Reading taken for the scale (the pages fix no
// rule): a block of 32 consecutive values gets 2^e with e the smallest
// integer such that max|x| <= 448 * 2^e (floored at -127, the smallest E8M0
// scale), so the block's largest magnitude lands in (224, 448] and nothing
// saturates; each value becomes x / 2^e (exact) rounded to the nearest e4m3
// value, ties to even.  The scale is stored as the E8M0 byte e + 127, the
// form the gfx950 scaled MFMA consumes.
#pragma once

#include "device.h"

namespace lcat {

constexpr int kFp8Block = 32;

// e for a block whose largest magnitude is amax (finite, >= 0): with
// amax = 1.m * 2^(E - 127), 448 * 2^e = 1.75 * 2^(e + 8).
__device__ __forceinline__ int fp8_block_exponent(float amax) {
  const uint32_t b = __builtin_bit_cast(uint32_t, amax);
  const int ef = (int)((b >> 23) & 0xFFu);
  const int e = (b & 0x7FFFFFu) <= 0x600000u ? ef - 135 : ef - 134;
  return e < -127 ? -127 : e;
}

// Four values, already divided by their block scale (|y| <= 448), into four
// e4m3 codes (one word, value i in byte i), round to nearest even.
__device__ __forceinline__ uint32_t fp8x4_rne(float y0, float y1, float y2, float y3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, lo, true);
}

}  // namespace lcat

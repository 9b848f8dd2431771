// Rotary-embedding angle arithmetic shared by the in-place RoPE kernel and
// the fused relayout + RoPE kernel, so both round identically.
//
// "Ulysses sequence parallelism in long-context inference", §3.2 and §5.3:
// RoPE is taken at each token's absolute position.  Reading for the formula
// (the pages print none): rotate-half pairing (i, i + D/2) with
// theta_i = base^(-2i/D).  Positions reach 2^17, where an fp32 angle would
// already be off by ~1e-2 rad, so the angle p * theta_i is formed in fp64 and
// reduced to [-pi, pi] with a two-constant Cody-Waite step (2*pi split into
// a double and its residual); sin/cos and the rotation then run in fp32 and
// the result is rounded to bf16 (nearest-even).
#pragma once

#include "device.h"

namespace lcat {

__device__ __forceinline__ double rope_theta(int i, int D, double log2_base) {
  return exp2(-(2.0 * i / D) * log2_base);
}

// (cos, sin) of position * theta
__device__ __forceinline__ float2 rope_cos_sin(double theta, int position) {
  const double two_pi_hi = 6.283185307179586;        // nearest double to 2*pi
  const double two_pi_lo = 2.4492935982947064e-16;   // 2*pi - two_pi_hi
  const double a = (double)position * theta;
  const double n = rint(a * (1.0 / two_pi_hi));
  double r = fma(-n, two_pi_hi, a);
  r = fma(-n, two_pi_lo, r);
  float sn, cn;
  sincosf((float)r, &sn, &cn);
  return make_float2(cn, sn);
}

// Rotate eight (x[i], x[i + D/2]) pairs held as two 8-element chunks.
__device__ __forceinline__ void rope_rotate8(const bf16x8 &lo, const bf16x8 &hi, const float2 *cs,
                                             bf16x8 &nlo, bf16x8 &nhi) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float2 f = cs[e];
    const float x0 = (float)lo[e], x1 = (float)hi[e];
    nlo[e] = to_bf16(fmaf(x0, f.x, -x1 * f.y));
    nhi[e] = to_bf16(fmaf(x1, f.x, x0 * f.y));
  }
}

}  // namespace lcat

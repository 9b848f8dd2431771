// Incoherent processing for the FP8 attention path: FA3's FP8 path ("Flash
// Attention and distributed inference", §18.5) pairs block quantisation with
// it, multiplying Q and K by one random orthogonal matrix before they are
// quantised, which leaves Q K^T unchanged and spreads large channels over
// all of them.  The pages name the step only.  Reading taken: each row x of
// 128 values becomes (s * x) H, H the Sylvester-Hadamard matrix (entries
// +-1, H[i][j] = (-1)^popcount(i & j)) and s the caller's signs; since
// H H^T = 128 I, (q M)(k M)^T = 128 q.k and the query multiplier takes the
// factor 1/128 (a power of two, exact).  The transform runs in fp32 as
// butterflies in a fixed order, span 1, 2, 4, ..., 64, element i with bit
// `span` clear pairing with i + span and the pair becoming (a + b, a - b),
// so its result (and the codes quantised from it) is reproducible bit for
// bit.
#pragma once

#include "device.h"
#include "kernels.h"

namespace lcat {

// v <- (s * v) H for one row of 128 values held by one lane.
__device__ __forceinline__ void hadamard128(float (&v)[128], const HadamardSigns &sg) {
#pragma unroll
  for (int i = 0; i < 128; ++i) {
    const uint32_t flip = ((sg.neg[i >> 5] >> (i & 31)) & 1u) << 31;
    v[i] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v[i]) ^ flip);
  }
#pragma unroll
  for (int span = 1; span < 128; span <<= 1) {
#pragma unroll
    for (int i = 0; i < 128; ++i) {
      if (i & span) continue;
      const float a = v[i], b = v[i + span];
      v[i] = a + b;
      v[i + span] = a - b;
    }
  }
}

}  // namespace lcat

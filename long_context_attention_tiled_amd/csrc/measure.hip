// Sustained bf16 MFMA rate of the device, as a yardstick for the prefill
// kernel besides the published dense peak.
//
// Every wave runs four independent accumulator chains of
// v_mfma_f32_32x32x16_bf16 on operands held in registers: no LDS, no memory
// traffic and almost no vector ALU work inside the loop, so the kernel shows
// the most any bf16 matrix kernel can reach on this part.  The operands are
// uniform random bf16 values in [-1, 1) (eight A and eight B sets per lane,
// rotated), because the rate depends on the data: with constant operands the
// matrix cores run at the nominal clock, while changing operands draw more
// power and the part slows its clock and its MFMA issue.  One workgroup of
// eight waves (two per SIMD) reserves enough LDS to own its CU.
#include <stdint.h>

#include "../../include/attn_measure.h"
#include "device.h"

namespace lcat {
namespace {

constexpr int kThreads = 512;
constexpr int kSets = 8;           // operand sets per lane
constexpr int kLdsPad = 100000;    // > half of a CU's 160 KiB: one workgroup per CU

__device__ __forceinline__ uint32_t xorshift32(uint32_t &h) {
  h ^= h << 13;
  h ^= h >> 17;
  h ^= h << 5;
  return h;
}

__device__ __forceinline__ __bf16 uniform_bf16(uint32_t &h) {
  return (__bf16)((float)(int)(xorshift32(h) & 0xffffu) * (1.0f / 32768.0f) - 1.0f);
}

__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(float *out, int iters, uint32_t seed) {
  __shared__ char pad[kLdsPad];
  const int tid = threadIdx.x;
  if (tid == 0) pad[blockIdx.x & 1023] = 0;
  uint32_t h = (blockIdx.x * (uint32_t)kThreads + tid) * 2654435761u + seed;
  if (h == 0) h = 1;   // xorshift has a fixed point at 0
  bf16x8 a[kSets], b[kSets];
#pragma unroll
  for (int s = 0; s < kSets; ++s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[s][i] = uniform_bf16(h);
      b[s][i] = uniform_bf16(h);
    }
  }
  f32x16 c[4] = {};
  // iters is a multiple of 4: each pass of the outer loop is 4 x 4 MFMAs
  for (int it = 0; it < iters; it += kSets / 2) {
#pragma unroll
    for (int s = 0; s < kSets; s += 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s + (i & 1)], b[(s + i) % kSets], c[i],
                                                       0, 0, 0);
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += c[i][r];
  __syncthreads();
  out[(long long)blockIdx.x * kThreads + tid] = sum + (float)pad[(tid * 7) & 1023];
}

}  // namespace
}  // namespace lcat

extern "C" int attn_measure_mfma_rate(float *out, int n_wg, int iters, uint32_t seed,
                                      void *stream) {
  if (!out) return ATTN_MEASURE_ERR_NULL;
  if (n_wg < 1 || n_wg > 65536 || iters < 4 || iters > (1 << 24) || iters % 4)
    return ATTN_MEASURE_ERR_SHAPE;
  hipLaunchKernelGGL(lcat::mfma_rate_kernel, dim3(n_wg), dim3(lcat::kThreads), 0,
                     static_cast<hipStream_t>(stream), out, iters, seed);
  return hipGetLastError() == hipSuccess ? ATTN_MEASURE_OK : ATTN_MEASURE_ERR_HIP;
}

// Block quantisation of bf16 rows into e4m3 codes with power-of-two scales
// (the rule is stated in fp8_block.h).  One thread per block of 32
// consecutive values: four 16-byte loads, the block maximum, then two
// 16-byte code stores and one scale byte.  Consecutive threads take
// consecutive blocks, so loads and stores are contiguous per wave.
#include "device.h"
#include "fp8_block.h"
#include "kernels.h"

namespace lcat {
namespace {

__global__ __launch_bounds__(256) void quantize_fp8_blocks_kernel(const bf16 *__restrict__ x,
                                                                  uint8_t *__restrict__ codes,
                                                                  uint8_t *__restrict__ scales,
                                                                  long long n_blocks) {
  const long long blk = (long long)blockIdx.x * 256 + threadIdx.x;
  if (blk >= n_blocks) return;
  const bf16 *src = x + blk * kFp8Block;
  bf16x8 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = as_bf16x8(ld_global_16(src + 8 * i));
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)v[i][e]));
  const int e = fp8_block_exponent(amax);
  u32x4 out[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = __builtin_amdgcn_ldexpf((float)v[i][k], -e);
    out[i >> 1][2 * (i & 1)] = fp8x4_rne(y[0], y[1], y[2], y[3]);
    out[i >> 1][2 * (i & 1) + 1] = fp8x4_rne(y[4], y[5], y[6], y[7]);
  }
  uint8_t *dst = codes + blk * kFp8Block;
  st_global_16(dst, out[0]);
  st_global_16(dst + 16, out[1]);
  scales[blk] = (uint8_t)(e + 127);
}

}  // namespace

hipError_t launch_quantize_fp8_blocks(const void *x, void *codes, uint8_t *scales,
                                      long long n_blocks, hipStream_t stream) {
  if (n_blocks <= 0) return hipSuccess;
  const long long n_wg = (n_blocks + 255) / 256;
  if (n_wg > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quantize_fp8_blocks_kernel, dim3((unsigned)n_wg), dim3(256), 0, stream,
                     static_cast<const bf16 *>(x), static_cast<uint8_t *>(codes), scales,
                     n_blocks);
  return hipGetLastError();
}

}  // namespace lcat

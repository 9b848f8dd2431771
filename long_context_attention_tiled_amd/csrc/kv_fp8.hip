// FP8 (OCP e4m3) copy of the paged KV cache with one fp32 scale per token.
//
// The Ulysses inference article (§5.4) keeps its KV cache quantised in
// groups; the format and grouping are a reading: e4m3 codes, one group per
// token's head vector (a K row, or a V column of the dimension-major V
// block), scale = amax / 448 so the largest element maps to the format's
// largest value 448.  Each element becomes x / scale rounded to the
// nearest e4m3 value (ties to even, magnitudes clamped to 448 first); an
// all-zero group gets scale 0 and codes 0.  The divisions are IEEE fp32
// divisions, so the codes are fixed by the definition.
//
// One workgroup (256 threads) per 64-token block.  K: four threads per token
// row, 32 elements each; the row maximum is combined with two lane
// exchanges.  V: two threads per dimension row, 32 keys each; the per-key
// (column) maximum is combined in LDS with an integer max on the float bits
// (magnitudes are non-negative, so their bit patterns order like their
// values).
#include "device.h"
#include "kernels.h"

namespace lcat {
namespace {

constexpr int HD = 128;
constexpr int BT = 64;
constexpr float kE4M3Max = 448.0f;

// Eight values already divided by their scale -> eight e4m3 codes (two words).
__device__ __forceinline__ u32x2 to_fp8x8(const float (&y)[8]) {
  u32x2 w;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) c[e] = fminf(fmaxf(y[4 * i + e], -kE4M3Max), kE4M3Max);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    w[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], lo, true);
  }
  return w;
}

__global__ __launch_bounds__(256) void kv_quantize_fp8_kernel(const bf16 *__restrict__ k_pool,
                                                              const bf16 *__restrict__ v_pool,
                                                              uint8_t *__restrict__ k8,
                                                              uint8_t *__restrict__ v8,
                                                              float *__restrict__ k_scale,
                                                              float *__restrict__ v_scale) {
  __shared__ uint32_t colmax[BT];
  const int tid = threadIdx.x;
  const size_t blk = blockIdx.x;
  if (tid < BT) colmax[tid] = 0u;

  // ---- K: token row j = tid / 4, elements 32 * (tid % 4) .. +31 ----------
  {
    const int j = tid >> 2, qd = tid & 3;
    const bf16 *src = k_pool + (blk * BT + j) * HD + 32 * qd;
    bf16x8 x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = as_bf16x8(ld_global_16(src + 8 * i));
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)x[i][e]));
    amax = fmaxf(amax, wave_shfl_xor(amax, 1));
    amax = fmaxf(amax, wave_shfl_xor(amax, 2));
    const float scale = amax / kE4M3Max;
    u32x4 out[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = scale > 0.f ? (float)x[i][e] / scale : 0.f;
      const u32x2 w = to_fp8x8(y);
      out[i >> 1][2 * (i & 1)] = w[0];
      out[i >> 1][2 * (i & 1) + 1] = w[1];
    }
    uint8_t *dst = k8 + (blk * BT + j) * HD + 32 * qd;
    st_global_16(dst, out[0]);
    st_global_16(dst + 16, out[1]);
    if (qd == 0) k_scale[blk * BT + j] = scale;
  }

  // ---- V: dimension row d = tid / 2, keys 32 * (tid % 2) .. +31 ----------
  __syncthreads();   // colmax cleared
  const int d = tid >> 1, hh = tid & 1;
  const bf16 *src = v_pool + (blk * HD + d) * BT + 32 * hh;
  bf16x8 x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = as_bf16x8(ld_global_16(src + 8 * i));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      atomicMax(&colmax[32 * hh + 8 * i + e], __builtin_bit_cast(uint32_t, fabsf((float)x[i][e])));
  __syncthreads();
  u32x4 out[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float scale = __builtin_bit_cast(float, colmax[32 * hh + 8 * i + e]) / kE4M3Max;
      y[e] = scale > 0.f ? (float)x[i][e] / scale : 0.f;
    }
    const u32x2 w = to_fp8x8(y);
    out[i >> 1][2 * (i & 1)] = w[0];
    out[i >> 1][2 * (i & 1) + 1] = w[1];
  }
  uint8_t *dst = v8 + (blk * HD + d) * BT + 32 * hh;
  st_global_16(dst, out[0]);
  st_global_16(dst + 16, out[1]);
  if (tid < BT) v_scale[blk * BT + tid] = __builtin_bit_cast(float, colmax[tid]) / kE4M3Max;
}

}  // namespace

hipError_t launch_kv_quantize_fp8(const void *k_pool, const void *v_pool, void *k8, void *v8,
                                  float *k_scale, float *v_scale, int n_blocks,
                                  hipStream_t stream) {
  if (n_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(kv_quantize_fp8_kernel, dim3(n_blocks), dim3(256), 0, stream,
                     static_cast<const bf16 *>(k_pool), static_cast<const bf16 *>(v_pool),
                     static_cast<uint8_t *>(k8), static_cast<uint8_t *>(v8), k_scale, v_scale);
  return hipGetLastError();
}

}  // namespace lcat

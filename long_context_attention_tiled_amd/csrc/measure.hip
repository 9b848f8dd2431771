// Yardsticks for the path's kernels, besides the published peaks: the
// sustained bf16 MFMA rate with operands in registers or with the A operand
// streamed from LDS (for prefill), and plain streaming HBM read and copy
// rates (for decode and the relayouts).
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
  out[(long long)blockIdx.x * kThreads + tid] = sum + (float)pad[blockIdx.x & 1023];
}

// The same chains with each MFMA's A operand read from LDS just before it
// (one 16-byte ds_read per lane per MFMA, as the attention kernels read K and
// V tiles): 64 KiB of random bf16 in LDS, each wave cycling through its own
// 8 KiB window; B operands from four register sets.  The LDS array plus a pad
// keep one workgroup per CU.
constexpr int kLdsBytes = 65536;
constexpr int kLdsPad2 = 40000;

__global__ __launch_bounds__(kThreads) void mfma_lds_rate_kernel(float *out, int iters,
                                                                 uint32_t seed) {
  __shared__ __attribute__((aligned(16))) char tile[kLdsBytes];
  __shared__ char pad[kLdsPad2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t h = (blockIdx.x * (uint32_t)kThreads + tid) * 2654435761u + seed;
  if (h == 0) h = 1;
  for (int i = tid; i < kLdsBytes / 2; i += kThreads) reinterpret_cast<__bf16 *>(tile)[i] = uniform_bf16(h);
  if (tid == 0) pad[blockIdx.x & 1023] = 0;
  bf16x8 b[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) b[s][i] = uniform_bf16(h);
  __syncthreads();
  f32x16 c[4] = {};
  const int base = wave * 8192 + lane * 16;   // 16-byte aligned, inside the tile
  int off = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(tile + base + off);
      off = (off + 1024) & 8191;
      c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[i], c[i], 0, 0, 0);
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += c[i][r];
  __syncthreads();
  out[(long long)blockIdx.x * kThreads + tid] = sum + (float)pad[blockIdx.x & 1023];
}

// Streaming read: wave w reads units [w * per_wave, (w + 1) * per_wave) of
// 16 bytes with non-temporal loads (the fastest way found to stream HBM on
// this part: 6.8-7.1 TB/s against 6.1-6.3 with plain loads), 32 loads per
// lane in flight, and folds them into one word per lane so the loads are
// live.
constexpr int kReadUnroll = 32;

__global__ __launch_bounds__(64) void hbm_read_kernel(const u32x4 *__restrict__ in,
                                                      uint32_t *out, long long per_wave) {
  const long long base = (long long)blockIdx.x * per_wave;
  u32x4 acc = {0, 0, 0, 0};
  for (long long u = threadIdx.x; u < per_wave; u += 64 * kReadUnroll) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int i = 0; i < kReadUnroll; ++i) {
      const long long x = u + 64LL * i;
      v[i] = x < per_wave ? __builtin_nontemporal_load(in + base + x) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kReadUnroll; ++i) acc ^= v[i];
  }
  out[(long long)blockIdx.x * 64 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Streaming copy of 16-byte units: 4 per thread, loads before stores,
// non-temporal loads and stores.
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

// in == out is allowed: each thread reads its units before it writes them.
__global__ __launch_bounds__(kCopyThreads) void hbm_copy_kernel(const u32x4 *in, u32x4 *out,
                                                               long long n_units) {
  const long long base = (long long)blockIdx.x * (kCopyThreads * kCopyUnroll) + threadIdx.x;
  u32x4 v[kCopyUnroll];
#pragma unroll
  for (int i = 0; i < kCopyUnroll; ++i) {
    const long long u = base + (long long)i * kCopyThreads;
    if (u < n_units) v[i] = __builtin_nontemporal_load(in + u);
  }
#pragma unroll
  for (int i = 0; i < kCopyUnroll; ++i) {
    const long long u = base + (long long)i * kCopyThreads;
    if (u < n_units) __builtin_nontemporal_store(v[i], out + u);
  }
}

}  // namespace
}  // namespace lcat

extern "C" long long attn_measure_hbm_read_bytes(long long bytes, int waves) {
  if (bytes < 16 || waves < 1 || waves > 65536) return 0;
  return (bytes / 16 / waves) * 16 * waves;
}

extern "C" int attn_measure_hbm_read(const void *buf, long long bytes, uint32_t *out, int waves,
                                     void *stream) {
  if (!buf || !out) return ATTN_MEASURE_ERR_NULL;
  if (waves < 1 || waves > 65536 || bytes / 16 < waves) return ATTN_MEASURE_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(buf) % 16) return ATTN_MEASURE_ERR_ALIGN;
  const long long per_wave = bytes / 16 / waves;
  hipLaunchKernelGGL(lcat::hbm_read_kernel, dim3(waves), dim3(64), 0,
                     static_cast<hipStream_t>(stream), static_cast<const lcat::u32x4 *>(buf), out,
                     per_wave);
  return hipGetLastError() == hipSuccess ? ATTN_MEASURE_OK : ATTN_MEASURE_ERR_HIP;
}

extern "C" int attn_measure_hbm_copy(const void *src, void *dst, long long bytes, void *stream) {
  if (!src || !dst) return ATTN_MEASURE_ERR_NULL;
  if (bytes < 16 || bytes % 16) return ATTN_MEASURE_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
    return ATTN_MEASURE_ERR_ALIGN;
  const char *s = static_cast<const char *>(src);
  const char *d = static_cast<const char *>(dst);
  if (s != d && s < d + bytes && d < s + bytes) return ATTN_MEASURE_ERR_SHAPE;   // overlap
  const long long n_units = bytes / 16;
  const long long per_wg = lcat::kCopyThreads * lcat::kCopyUnroll;
  const long long n_wg = (n_units + per_wg - 1) / per_wg;
  if (n_wg > 0x7fffffffLL) return ATTN_MEASURE_ERR_SHAPE;
  hipLaunchKernelGGL(lcat::hbm_copy_kernel, dim3((unsigned)n_wg), dim3(lcat::kCopyThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const lcat::u32x4 *>(src),
                     static_cast<lcat::u32x4 *>(dst), n_units);
  return hipGetLastError() == hipSuccess ? ATTN_MEASURE_OK : ATTN_MEASURE_ERR_HIP;
}

extern "C" int attn_measure_mfma_rate(float *out, int n_wg, int iters, uint32_t seed,
                                      int a_from_lds, void *stream) {
  if (!out) return ATTN_MEASURE_ERR_NULL;
  if (n_wg < 1 || n_wg > 65536 || iters < 4 || iters > (1 << 24) || iters % 4 ||
      (a_from_lds != 0 && a_from_lds != 1))
    return ATTN_MEASURE_ERR_SHAPE;
  if (a_from_lds)
    hipLaunchKernelGGL(lcat::mfma_lds_rate_kernel, dim3(n_wg), dim3(lcat::kThreads), 0,
                       static_cast<hipStream_t>(stream), out, iters, seed);
  else
    hipLaunchKernelGGL(lcat::mfma_rate_kernel, dim3(n_wg), dim3(lcat::kThreads), 0,
                       static_cast<hipStream_t>(stream), out, iters, seed);
  return hipGetLastError() == hipSuccess ? ATTN_MEASURE_OK : ATTN_MEASURE_ERR_HIP;
}

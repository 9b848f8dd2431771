// Block quantisation of bf16 rows into e4m3 codes with power-of-two scales
// (the rule is stated in fp8_block.h).  Four consecutive threads share a
// block of 32 consecutive values, 8 each: one 16-byte load per thread (a
// wave reads 1 KiB contiguous), the block maximum across the four lanes,
// then an 8-byte code store per thread and one scale byte per block.
#include "device.h"
#include "fp8_block.h"
#include "hadamard.h"
#include "kernels.h"

namespace lcat {
namespace {

__global__ __launch_bounds__(256) void quantize_fp8_blocks_kernel(const bf16 *__restrict__ x,
                                                                  uint8_t *__restrict__ codes,
                                                                  uint8_t *__restrict__ scales,
                                                                  long long n_blocks) {
  const long long q = (long long)blockIdx.x * 256 + threadIdx.x;   // quarter block
  const bool live = q < 4 * n_blocks;                              // n_blocks * 4 quarters
  const bf16x8 v = live ? as_bf16x8(ld_global_16_nt(x + 8 * q)) : bf16x8{};
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf((float)v[k]));
  // the four lanes of a block are consecutive lanes of one wave
  amax = fmaxf(amax, wave_shfl_xor(amax, 1));
  amax = fmaxf(amax, wave_shfl_xor(amax, 2));
  if (!live) return;
  const int e = fp8_block_exponent(amax);
  float y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = __builtin_amdgcn_ldexpf((float)v[k], -e);
  const uint32_t lo = fp8x4_rne(y[0], y[1], y[2], y[3]), hi = fp8x4_rne(y[4], y[5], y[6], y[7]);
  *reinterpret_cast<uint2 *>(codes + 8 * q) = make_uint2(lo, hi);
  if ((q & 3) == 0) scales[q >> 2] = (uint8_t)(e + 127);
}

// Rows of 128 rotated by (s * x) H (hadamard.h) and then block-quantised
// as above: one thread per row (the transform needs the whole row), 256
// bytes in, 128 code bytes and the row's 4 scale bytes out.
__global__ __launch_bounds__(256) void quantize_fp8_rotated_kernel(const bf16 *__restrict__ x,
                                                                   uint8_t *__restrict__ codes,
                                                                   uint8_t *__restrict__ scales,
                                                                   long long n_rows, HadamardSigns sg) {
  const long long row = (long long)blockIdx.x * 256 + threadIdx.x;
  if (row >= n_rows) return;
  const bf16 *src = x + row * 128;
  float v[128];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bf16x8 raw = as_bf16x8(ld_global_16(src + 8 * i));
#pragma unroll
    for (int e = 0; e < 8; ++e) v[8 * i + e] = (float)raw[e];
  }
  hadamard128(v, sg);
  uint32_t sc = 0;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[32 * blk + i]));
    const int e = fp8_block_exponent(amax);
    sc |= (uint32_t)(e + 127) << (8 * blk);
    u32x4 out[2];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const float *y = v + 32 * blk + 4 * w;
      out[w >> 2][w & 3] = fp8x4_rne(__builtin_amdgcn_ldexpf(y[0], -e), __builtin_amdgcn_ldexpf(y[1], -e),
                                     __builtin_amdgcn_ldexpf(y[2], -e), __builtin_amdgcn_ldexpf(y[3], -e));
    }
    uint8_t *dst = codes + row * 128 + 32 * blk;
    st_global_16(dst, out[0]);
    st_global_16(dst + 16, out[1]);
  }
  *reinterpret_cast<uint32_t *>(scales + row * 4) = sc;
}

// V for FP8 P V: blocks run along keys (the contraction axis of P V).  One
// workgroup per (batch, KV head, 64-key tile): the 64 x 128 bf16 tile comes
// in with 16-byte loads (16 threads per 256-byte key row) and is written to
// LDS key-major as 4-byte words, rows 65 words apart; thread (d, h) then
// reads the 32 keys 32 h .. +31 of dim d down a column (the pitch puts the
// rows of the two key halves 32 banks apart, and the lanes of a wave on
// distinct words, so neither side has bank conflicts), quantises them as one
// block and writes their 32 codes, so the two threads of a dim write its 64
// contiguous codes.
// Output: v8t [B][Hkv][128][S64] (dimension-major, S64 = S rounded up to 64,
// keys >= S written as code 0) and per 64-key tile a 256-byte scale block
// whose byte 4 (32 h + r) + db is the scale of dim 32 db + r over keys
// 64 t + 32 h .. +31: the word lane r + 32 h of a wave loads is the A-operand
// scale word of P V for that lane, one dim group db per byte.
constexpr int kVqPitch = 65;   // LDS row (one key) in 4-byte words: 64 words of dims + pad
__global__ __launch_bounds__(256) void quantize_fp8_v_kernel(const bf16 *__restrict__ v,
                                                             uint8_t *__restrict__ v8t,
                                                             uint8_t *__restrict__ v_scale, int S,
                                                             int Hkv, int S64) {
  __shared__ uint32_t tile[64 * kVqPitch];
  const int tid = threadIdx.x;
  const int n_tiles = S64 / 64;
  const int t = blockIdx.x % n_tiles;
  const long long bg = blockIdx.x / n_tiles;   // b * Hkv + g
  const long long b = bg / Hkv;
  const int g = (int)(bg % Hkv);
  const int key0 = 64 * t;
  // load: chunk c = tid + 256 u covers key c / 16, dims 8 (c % 16) .. +7
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = tid + 256 * u;
    const int key = c >> 4, w0 = 4 * (c & 15);
    u32x4 x = {};
    if (key0 + key < S)
      x = ld_global_16_nt(v + (((b * S + key0 + key) * Hkv + g) * 128 + 2 * w0));
#pragma unroll
    for (int w = 0; w < 4; ++w) tile[key * kVqPitch + w0 + w] = x[w];
  }
  __syncthreads();
  const int d = tid >> 1, h = tid & 1;
  const int half_sel = 16 * (d & 1);   // dim d is the low (even d) or high half of word d / 2
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t wd = tile[(32 * h + i) * kVqPitch + (d >> 1)];
    x[i] = __builtin_bit_cast(float, (wd >> half_sel) << 16);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const int e = fp8_block_exponent(amax);
  u32x4 out[2];
#pragma unroll
  for (int w = 0; w < 8; ++w)
    out[w >> 2][w & 3] = fp8x4_rne(__builtin_amdgcn_ldexpf(x[4 * w], -e), __builtin_amdgcn_ldexpf(x[4 * w + 1], -e),
                                   __builtin_amdgcn_ldexpf(x[4 * w + 2], -e), __builtin_amdgcn_ldexpf(x[4 * w + 3], -e));
  uint8_t *dst = v8t + (bg * 128 + d) * (long long)S64 + key0 + 32 * h;
  st_global_16(dst, out[0]);
  st_global_16(dst + 16, out[1]);
  v_scale[(bg * n_tiles + t) * 256 + 4 * (32 * h + (d & 31)) + (d >> 5)] = (uint8_t)(e + 127);
}

}  // namespace

hipError_t launch_quantize_fp8_blocks(const void *x, void *codes, uint8_t *scales,
                                      long long n_blocks, hipStream_t stream) {
  if (n_blocks <= 0) return hipSuccess;
  const long long n_wg = (4 * n_blocks + 255) / 256;
  if (n_wg > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quantize_fp8_blocks_kernel, dim3((unsigned)n_wg), dim3(256), 0, stream,
                     static_cast<const bf16 *>(x), static_cast<uint8_t *>(codes), scales,
                     n_blocks);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8_rotated(const void *x, void *codes, uint8_t *scales,
                                       long long n_rows, HadamardSigns sg, hipStream_t stream) {
  if (n_rows <= 0) return hipSuccess;
  const long long n_wg = (n_rows + 255) / 256;
  if (n_wg > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quantize_fp8_rotated_kernel, dim3((unsigned)n_wg), dim3(256), 0, stream,
                     static_cast<const bf16 *>(x), static_cast<uint8_t *>(codes), scales, n_rows, sg);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8_v(const void *v, void *v8t, uint8_t *v_scale, int B, int S, int Hkv,
                                 hipStream_t stream) {
  const int S64 = (S + 63) / 64 * 64;
  const long long n_wg = (long long)B * Hkv * (S64 / 64);
  if (n_wg <= 0) return hipSuccess;
  if (n_wg > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quantize_fp8_v_kernel, dim3((unsigned)n_wg), dim3(256), 0, stream,
                     static_cast<const bf16 *>(v), static_cast<uint8_t *>(v8t), v_scale, S, Hkv, S64);
  return hipGetLastError();
}

}  // namespace lcat

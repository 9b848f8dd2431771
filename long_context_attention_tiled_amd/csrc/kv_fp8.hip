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
// One workgroup (256 threads) per 64-token block; the K and V loads of a
// thread are issued together at the start.  K: four threads per token row,
// 32 elements each; the row maximum is combined with two lane exchanges.
// V: two threads per dimension row, 32 keys each.  The per-key (column)
// maximum goes through LDS: the magnitudes, as bf16 bit patterns (sign
// cleared; non-negative patterns order like their values), are written as
// a [128][64] tile, each thread takes the maximum of a pair of keys over 16
// dimensions with packed 16-bit integer maxima, and 64 threads fold the 8
// partial maxima of their key.
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

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256) void kv_quantize_fp8_kernel(const bf16 *__restrict__ k_pool,
                                                              const bf16 *__restrict__ v_pool,
                                                              uint8_t *__restrict__ k8,
                                                              uint8_t *__restrict__ v8,
                                                              float *__restrict__ k_scale,
                                                              float *__restrict__ v_scale) {
  constexpr int PITCH = BT / 2 + 1;            // dwords per dimension row of the tile
  __shared__ uint32_t vmag[HD * PITCH];        // |V| as bf16 pairs: [d][key pair]
  __shared__ uint32_t part[8][BT / 2];         // column maxima over 16 dims, key pairs
  __shared__ float vsc[BT];
  const int tid = threadIdx.x;
  const size_t blk = blockIdx.x;

  // K: token row j = tid / 4, elements 32 * (tid % 4) .. +31;
  // V: dimension row d = tid / 2, keys 32 * (tid % 2) .. +31
  const int j = tid >> 2, qd = tid & 3;
  const int d = tid >> 1, hh = tid & 1;
  const bf16 *ksrc = k_pool + (blk * BT + j) * HD + 32 * qd;
  const bf16 *vsrc = v_pool + (blk * HD + d) * BT + 32 * hh;
  bf16x8 kx[4], vx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kx[i] = as_bf16x8(ld_global_16(ksrc + 8 * i));
#pragma unroll
  for (int i = 0; i < 4; ++i) vx[i] = as_bf16x8(ld_global_16(vsrc + 8 * i));

  // ---- V magnitudes into the tile (read back after the K part) ----------
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int w = 0; w < 4; ++w)
      vmag[d * PITCH + 16 * hh + 4 * i + w] = as_u32x4(vx[i])[w] & 0x7FFF7FFFu;

  // ---- K ------------------------------------------------------------------
  {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)kx[i][e]));
    amax = fmaxf(amax, wave_shfl_xor(amax, 1));
    amax = fmaxf(amax, wave_shfl_xor(amax, 2));
    const float scale = amax / kE4M3Max;
    u32x4 out[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = scale > 0.f ? (float)kx[i][e] / scale : 0.f;
      const u32x2 w = to_fp8x8(y);
      out[i >> 1][2 * (i & 1)] = w[0];
      out[i >> 1][2 * (i & 1) + 1] = w[1];
    }
    uint8_t *dst = k8 + (blk * BT + j) * HD + 32 * qd;
    st_global_16(dst, out[0]);
    st_global_16(dst + 16, out[1]);
    if (qd == 0) k_scale[blk * BT + j] = scale;
  }

  // ---- V column maxima: thread (dims 16 g .., key pair kp) ----------------
  __syncthreads();
  {
    const int kp = tid & 31, g = tid >> 5;
    u16x2 m = {0, 0};
#pragma unroll
    for (int r = 0; r < 16; ++r)
      m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, vmag[(16 * g + r) * PITCH + kp]));
    part[g][kp] = __builtin_bit_cast(uint32_t, m);
  }
  __syncthreads();
  if (tid < BT) {
    uint32_t m = 0;
#pragma unroll
    for (int g = 0; g < 8; ++g) m = max(m, (part[g][tid >> 1] >> (16 * (tid & 1))) & 0xFFFFu);
    const float scale = __builtin_bit_cast(float, m << 16) / kE4M3Max;
    vsc[tid] = scale;
    v_scale[blk * BT + tid] = scale;
  }
  __syncthreads();

  // ---- V codes ------------------------------------------------------------
  u32x4 out[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float scale = vsc[32 * hh + 8 * i + e];
      y[e] = scale > 0.f ? (float)vx[i][e] / scale : 0.f;
    }
    const u32x2 w = to_fp8x8(y);
    out[i >> 1][2 * (i & 1)] = w[0];
    out[i >> 1][2 * (i & 1) + 1] = w[1];
  }
  uint8_t *dst = v8 + (blk * HD + d) * BT + 32 * hh;
  st_global_16(dst, out[0]);
  st_global_16(dst + 16, out[1]);
}

// Append T new tokens per request straight into the fp8 pools (the token ->
// slot map of attn_kv_append), quantising each token's K row and V vector
// with its own scale exactly as the pool quantiser does.  One workgroup per
// (touched block, KV head, request); four threads per token, 32 elements
// each.  The V codes are staged in LDS and written dimension row by
// dimension row, one byte per lane (consecutive slots), so earlier tokens of
// a partially filled block are left as they are.
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(
    const bf16 *__restrict__ k_new, const bf16 *__restrict__ v_new, uint8_t *__restrict__ k8,
    uint8_t *__restrict__ v8, float *__restrict__ k_scale, float *__restrict__ v_scale,
    int n_blocks, const int32_t *__restrict__ block_head, const int32_t *__restrict__ block_table,
    int max_blocks, const int32_t *__restrict__ start_pos, int T, int Hkv, int kv_head_base,
    int32_t *dev_status) {
  __shared__ uint8_t vcodes[BT * (HD + 4)];   // [slot][dim], rows padded by 4 bytes
  const int tid = threadIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  const int start = start_pos[b];
  if (start < 0 || (long long)start + T > (long long)max_blocks * BT) {
    if (blockIdx.x == 0 && tid == 0 && dev_status) dev_status[0] = 2;
    return;
  }
  const int j = start / BT + (int)blockIdx.x;          // logical block of this workgroup
  const int lo = max(start, j * BT), hi = min(start + T, (j + 1) * BT);
  if (lo >= hi) return;
  const int blk = block_table[((size_t)b * Hkv + g) * max_blocks + j];
  if (blk < 0 || blk >= n_blocks) {
    if (tid == 0 && dev_status) dev_status[0] = 2;
    return;
  }
  if (block_head[blk] != kv_head_base + g) {
    if (tid == 0 && dev_status) dev_status[0] = 1;
    return;
  }
  const int s_lo = lo - j * BT, s_hi = hi - j * BT;     // slot range [s_lo, s_hi)
  const int slot = tid >> 2, qd = tid & 3;
  const bool live = slot >= s_lo && slot < s_hi;        // uniform over each group of 4 lanes
  const size_t src = live ? (((size_t)b * T + (j * BT + slot - start)) * Hkv + g) * HD + 32 * qd : 0;
  for (int which = 0; which < 2; ++which) {
    const bf16 *in = which == 0 ? k_new : v_new;
    bf16x8 x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = live ? as_bf16x8(ld_global_16(in + src + 8 * i)) : bf16x8{};
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
    if (which == 0) {
      if (live) {
        uint8_t *dst = k8 + ((size_t)blk * BT + slot) * HD + 32 * qd;
        st_global_16(dst, out[0]);
        st_global_16(dst + 16, out[1]);
        if (qd == 0) k_scale[(size_t)blk * BT + slot] = scale;
      }
    } else {
      uint32_t *row = reinterpret_cast<uint32_t *>(vcodes + slot * (HD + 4) + 32 * qd);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        row[e] = out[0][e];
        row[4 + e] = out[1][e];
      }
      if (live && qd == 0) v_scale[(size_t)blk * BT + slot] = scale;
    }
  }
  __syncthreads();
  // V^T rows: lane = slot, each wave walks a quarter of the dimensions
  const int ls = tid & 63;
  if (ls >= s_lo && ls < s_hi) {
    uint8_t *dst = v8 + (size_t)blk * HD * BT + ls;
    for (int d = tid >> 6; d < HD; d += 4) dst[(size_t)d * BT] = vcodes[ls * (HD + 4) + d];
  }
}

}  // namespace

hipError_t launch_kv_append_fp8(const void *k_new, const void *v_new, void *k8, void *v8,
                                float *k_scale, float *v_scale, int n_blocks,
                                const int32_t *block_head, const int32_t *block_table,
                                int max_blocks, const int32_t *start_pos, int T, int B, int Hkv,
                                int kv_head_base, int32_t *dev_status, hipStream_t stream) {
  if (T <= 0 || B <= 0) return hipSuccess;
  dim3 grid((T + BT - 1) / BT + 1, Hkv, B), block(256);
  hipLaunchKernelGGL(kv_append_fp8_kernel, grid, block, 0, stream,
                     static_cast<const bf16 *>(k_new), static_cast<const bf16 *>(v_new),
                     static_cast<uint8_t *>(k8), static_cast<uint8_t *>(v8), k_scale, v_scale,
                     n_blocks, block_head, block_table, max_blocks, start_pos, T, Hkv,
                     kv_head_base, dev_status);
  return hipGetLastError();
}

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

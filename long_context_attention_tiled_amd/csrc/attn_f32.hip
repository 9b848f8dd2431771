// Exact attention with fp32 inputs and fp32 arithmetic throughout.
//
// Same computation as the bf16 path ("Flash Attention and distributed
// inference", §18.2 definition, §18.3 tiled online softmax with rescaling,
// §18.4 final division), kept in fp32 end to end so that small fp32 problems
// meet a 1e-3 absolute bound without any bf16 rounding.  One thread owns one
// query row (its q vector and output accumulator live in registers); the
// workgroup stages 32-key K/V tiles in LDS and every thread reads them with
// broadcast loads.
#include "device.h"
#include "kernels.h"

namespace lcat {
namespace {

constexpr int TK = 32;   // keys per LDS tile
constexpr int QB = 64;   // query rows per workgroup

template <int D, bool CAUSAL>
__global__ __launch_bounds__(QB) void attn_f32_kernel(const float *__restrict__ q,
                                                      const float *__restrict__ k,
                                                      const float *__restrict__ v,
                                                      float *__restrict__ o, float *__restrict__ lse,
                                                      int S, int Hq, int Hkv, float scale) {
  __shared__ float ks[TK][D];
  __shared__ float vs[TK][D];
  const int tid = threadIdx.x;
  const int qblk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (Hq / Hkv);
  const int row = qblk * QB + tid;
  const bool valid = row < S;

  float qr[D], acc[D];
  const float *qsrc = q + (((size_t)b * S + (valid ? row : 0)) * Hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = valid ? qsrc[d] : 0.f;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int last_row = min(qblk * QB + QB - 1, S - 1);
  const int n_keys = CAUSAL ? last_row + 1 : S;

  for (int k0 = 0; k0 < n_keys; k0 += TK) {
    __syncthreads();
    for (int idx = tid; idx < TK * D; idx += QB) {
      const int kk = idx / D, d = idx % D;
      const int key = k0 + kk;
      const size_t off = (((size_t)b * S + key) * Hkv + g) * D + d;
      ks[kk][d] = key < S ? k[off] : 0.f;
      vs[kk][d] = key < S ? v[off] : 0.f;
    }
    __syncthreads();

    float s[TK];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      const int key = k0 + kk;
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(qr[d], ks[kk][d], dot);
      const bool ok = key < S && (!CAUSAL || key <= row);
      s[kk] = ok ? dot * scale : -INFINITY;
      mx = fmaxf(mx, s[kk]);
    }
    const float m_new = fmaxf(m, mx);
    if (m_new == -INFINITY) continue;   // nothing visible yet for this row
    const float alpha = expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      const float pk = expf(s[kk] - m_new);
      l += pk;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(pk, vs[kk][d], acc[d]);
    }
    m = m_new;
  }

  if (valid) {
    const float inv = 1.f / l;
    float *dst = o + (((size_t)b * S + row) * Hq + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) dst[d] = acc[d] * inv;
    if (lse) lse[((size_t)b * Hq + h) * S + row] = m + logf(l);
  }
}

template <int D>
hipError_t launch_d(const float *q, const float *k, const float *v, float *o, float *lse, int B,
                    int S, int Hq, int Hkv, int causal, float scale, hipStream_t stream) {
  dim3 grid((S + QB - 1) / QB, Hq, B), block(QB);
  if (causal)
    hipLaunchKernelGGL((attn_f32_kernel<D, true>), grid, block, 0, stream, q, k, v, o, lse, S, Hq,
                       Hkv, scale);
  else
    hipLaunchKernelGGL((attn_f32_kernel<D, false>), grid, block, 0, stream, q, k, v, o, lse, S,
                       Hq, Hkv, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                           int B, int S, int Hq, int Hkv, int D, int causal, float scale,
                           hipStream_t stream) {
  if (D == 64) return launch_d<64>(q, k, v, o, lse, B, S, Hq, Hkv, causal, scale, stream);
  if (D == 128) return launch_d<128>(q, k, v, o, lse, B, S, Hq, Hkv, causal, scale, stream);
  return hipErrorInvalidValue;
}

}  // namespace lcat

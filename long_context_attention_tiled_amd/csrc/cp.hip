// Context parallelism on one GPU ("LLM推理中的多卡切分", §3.5 and §3.5.1):
// the sequence is split over N ranks (contiguous blocks for ring attention,
// round-robin stripes, or the zigzag / in-seq-split pairing of blocks i and
// 2N-1-i), each rank computes its queries against every rank's key shard,
// and the partial results are combined with the log-sum-exp rescale.
//
// This file holds the data movement and bookkeeping around the attention
// kernel: gathering one rank's tokens out of the full sequence (and
// scattering results back), turning two ascending position lists into
// per-row key counts for the prefix-limited attention, and merging two
// normalised partial results (O, LSE).
#include "device.h"
#include "kernels.h"

namespace lcat {
namespace {

constexpr int NT = 256;
constexpr int UPT = 4;   // 16-byte units per thread

// Local token i of the shard is global token
//   i < len_a ? start_a + i * stride : start_b + (i - len_a) * stride
__device__ __forceinline__ long long shard_token(const CpMap &m, long long i) {
  return i < m.len_a ? m.start_a + i * m.stride : m.start_b + (i - m.len_a) * m.stride;
}

// Shard copy in 16-byte units: unit u of the shard side belongs to local token
// u / units_per_tok.  scatter = 0: full -> shard (gather), 1: shard -> full.
__global__ __launch_bounds__(NT) void cp_copy16_kernel(const char *__restrict__ in,
                                                       char *__restrict__ out, CpMap m,
                                                       long long n_units, int units_per_tok,
                                                       int scatter, int32_t *positions) {
  const long long base = (long long)blockIdx.x * (NT * UPT) + threadIdx.x;
  u32x4 buf[UPT];
  long long full[UPT];
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const long long u = base + (long long)k * NT;
    const long long i = u / units_per_tok;
    const int w = (int)(u - i * units_per_tok);
    full[k] = (shard_token(m, i) * units_per_tok + w) * 16;
    if (positions && w == 0 && u < n_units) positions[i] = (int32_t)shard_token(m, i);
  }
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const long long u = base + (long long)k * NT;
    if (u < n_units) buf[k] = ld_global_16(in + (scatter ? 16 * u : full[k]));
  }
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const long long u = base + (long long)k * NT;
    if (u < n_units)
      __builtin_nontemporal_store(buf[k], reinterpret_cast<u32x4 *>(out + (scatter ? full[k] : 16 * u)));
  }
}

// Element-wise fallback for rows that are not whole 16-byte units.
__global__ __launch_bounds__(NT) void cp_copy_elem_kernel(const char *__restrict__ in,
                                                          char *__restrict__ out, CpMap m,
                                                          long long n_bytes, int row_bytes,
                                                          int scatter, int32_t *positions) {
  const long long e = (long long)blockIdx.x * NT + threadIdx.x;
  if (e >= n_bytes) return;
  const long long i = e / row_bytes;
  const int w = (int)(e - i * row_bytes);
  const long long full = shard_token(m, i) * row_bytes + w;
  if (positions && w == 0) positions[i] = (int32_t)shard_token(m, i);
  if (scatter)
    out[full] = in[e];
  else
    out[e] = in[full];
}

// lim[b][i] = number of keys of batch b whose position is <= q_pos[b][i]
// (k_pos ascending): an upper-bound binary search per query row.
__global__ __launch_bounds__(NT) void key_limits_kernel(const int32_t *__restrict__ q_pos,
                                                        const int32_t *__restrict__ k_pos,
                                                        int32_t *__restrict__ lim, int B, int Sq,
                                                        int Sk) {
  const long long r = (long long)blockIdx.x * NT + threadIdx.x;
  if (r >= (long long)B * Sq) return;
  const int b = (int)(r / Sq);
  const int32_t p = q_pos[r];
  const int32_t *kp = k_pos + (size_t)b * Sk;
  int lo = 0, hi = Sk;   // first index with kp > p lies in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (kp[mid] <= p)
      lo = mid + 1;
    else
      hi = mid;
  }
  lim[r] = lo;
}

// Merge of two normalised partials of the same rows over disjoint key sets:
//   M = max(la, lb), wa = e^(la-M), wb = e^(lb-M),
//   O = (wa Oa + wb Ob) / (wa + wb), LSE = M + ln(wa + wb);
// a side with LSE = -inf has weight 0, and if both do, O = 0, LSE = -inf.
// One 16-byte unit (8 bf16) of O per thread; O [B][S][H][D], LSE [B][H][S].
__global__ __launch_bounds__(NT) void merge_kernel(const bf16 *oa, const float *la, const bf16 *ob,
                                                   const float *lb, bf16 *o, float *lse, int B,
                                                   int S, int H, int D) {
  const int upr = D / 8;   // units per row
  const long long u = (long long)blockIdx.x * NT + threadIdx.x;
  if (u >= (long long)B * S * H * upr) return;
  const long long row = u / upr;   // (b, s, h)
  const int w = (int)(u - row * upr);
  const int h = (int)(row % H);
  const long long bs = row / H;
  const int s = (int)(bs % S), b = (int)(bs / S);
  const size_t li = ((size_t)b * H + h) * S + s;
  const float a = la[li], c = lb[li];
  const float M = fmaxf(a, c);
  float wa = 0.f, wc = 0.f;
  if (M != -INFINITY) {
    wa = a == -INFINITY ? 0.f : expf(a - M);
    wc = c == -INFINITY ? 0.f : expf(c - M);
  }
  const float den = wa + wc;
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const bf16x8 xa = as_bf16x8(ld_global_16(oa + row * D + 8 * w));
  const bf16x8 xc = as_bf16x8(ld_global_16(ob + row * D + 8 * w));
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float va = wa > 0.f ? (float)xa[e] : 0.f;
    const float vc = wc > 0.f ? (float)xc[e] : 0.f;
    r[e] = to_bf16((wa * va + wc * vc) * inv);
  }
  st_global_16(o + row * D + 8 * w, as_u32x4(r));
  if (w == 0 && lse) lse[li] = den > 0.f ? M + logf(den) : -INFINITY;
}

}  // namespace

hipError_t launch_cp_copy(const void *in, void *out, const CpMap &m, long long n_tok,
                          long long row_bytes, int scatter, int32_t *positions,
                          hipStream_t stream) {
  if (n_tok == 0) return hipSuccess;
  const bool v16 = row_bytes % 16 == 0 && reinterpret_cast<uintptr_t>(in) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(out) % 16 == 0;
  if (v16) {
    const int upt = (int)(row_bytes / 16);
    const long long n_units = n_tok * upt;
    const long long n_wg = (n_units + NT * UPT - 1) / (NT * UPT);
    hipLaunchKernelGGL(cp_copy16_kernel, dim3((unsigned)n_wg), dim3(NT), 0, stream,
                       static_cast<const char *>(in), static_cast<char *>(out), m, n_units, upt,
                       scatter, positions);
  } else {
    const long long n_bytes = n_tok * row_bytes;
    const long long n_wg = (n_bytes + NT - 1) / NT;
    hipLaunchKernelGGL(cp_copy_elem_kernel, dim3((unsigned)n_wg), dim3(NT), 0, stream,
                       static_cast<const char *>(in), static_cast<char *>(out), m, n_bytes,
                       (int)row_bytes, scatter, positions);
  }
  return hipGetLastError();
}

hipError_t launch_key_limits(const int32_t *q_pos, const int32_t *k_pos, int32_t *lim, int B,
                             int Sq, int Sk, hipStream_t stream) {
  const long long n = (long long)B * Sq;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(key_limits_kernel, dim3((unsigned)((n + NT - 1) / NT)), dim3(NT), 0, stream,
                     q_pos, k_pos, lim, B, Sq, Sk);
  return hipGetLastError();
}

hipError_t launch_merge(const void *oa, const float *la, const void *ob, const float *lb, void *o,
                        float *lse, int B, int S, int H, int D, hipStream_t stream) {
  const long long n = (long long)B * S * H * (D / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((n + NT - 1) / NT)), dim3(NT), 0, stream,
                     static_cast<const bf16 *>(oa), la, static_cast<const bf16 *>(ob), lb,
                     static_cast<bf16 *>(o), lse, B, S, H, D);
  return hipGetLastError();
}

}  // namespace lcat

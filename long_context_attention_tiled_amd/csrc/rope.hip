// Rotary position embedding at absolute token positions, in place.
//
// "Ulysses sequence parallelism in long-context inference", §3.2: every
// local token is bound to its position in the original sequence through a
// global token index table and RoPE is generated from that absolute
// position; §5.3 describes the failure when local indices are used instead.
// Reading taken for the formula (the pages do not print one): rotate-half
// pairing (i, i + D/2) with theta_i = base^(-2i/D).
//
// Precision: positions reach 2^17, where an fp32 angle would already be off
// by ~1e-2 rad.  The angle p * theta_i is therefore formed in fp64 and
// reduced to [-pi, pi] with a two-constant Cody-Waite step (2*pi split into
// a double and its residual), then sin/cos and the rotation run in fp32 and
// the result is rounded to bf16 (nearest-even).
//
// A workgroup handles a few consecutive tokens: it first builds the
// (cos, sin) table of those tokens in LDS (each angle once, shared by all
// heads), then streams the heads with 16-byte loads and stores.
#include "device.h"
#include "kernels.h"

namespace lcat {
namespace {

constexpr int NT = 256;
constexpr int MAX_TABLE = 4096;   // (token, frequency) pairs per workgroup

__global__ __launch_bounds__(NT) void rope_kernel(bf16 *__restrict__ x,
                                                  const int32_t *__restrict__ positions, int S,
                                                  int H, int D, double log2_base, int tok_per_wg) {
  __shared__ float2 cs[MAX_TABLE];
  const int tid = threadIdx.x;
  const int half = D >> 1;
  const int t0 = blockIdx.x * tok_per_wg;
  const int nt = min(tok_per_wg, S - t0);
  if (nt <= 0) return;

  const double two_pi_hi = 6.283185307179586;        // nearest double to 2*pi
  const double two_pi_lo = 2.4492935982947064e-16;   // 2*pi - two_pi_hi
  for (int idx = tid; idx < nt * half; idx += NT) {
    const int t = idx / half, i = idx % half;
    const double theta = exp2(-(2.0 * i / D) * log2_base);
    const double a = (double)positions[t0 + t] * theta;
    const double n = rint(a * (1.0 / two_pi_hi));
    double r = fma(-n, two_pi_hi, a);
    r = fma(-n, two_pi_lo, r);
    float sn, cn;
    sincosf((float)r, &sn, &cn);
    cs[idx] = make_float2(cn, sn);
  }
  __syncthreads();

  const int chunks = half >> 3;                      // 8-element chunks per half
  const int items = nt * H * chunks;
  for (int it = tid; it < items; it += NT) {
    const int c = it % chunks;
    const int th = it / chunks;
    const int h = th % H, t = th / H;
    bf16 *row = x + ((size_t)(t0 + t) * H + h) * D;
    const bf16x8 lo = as_bf16x8(ld_global_16(row + 8 * c));
    const bf16x8 hi = as_bf16x8(ld_global_16(row + half + 8 * c));
    bf16x8 nlo, nhi;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 f = cs[t * half + 8 * c + e];
      const float x0 = (float)lo[e], x1 = (float)hi[e];
      nlo[e] = to_bf16(fmaf(x0, f.x, -x1 * f.y));
      nhi[e] = to_bf16(fmaf(x1, f.x, x0 * f.y));
    }
    st_global_16(row + 8 * c, as_u32x4(nlo));
    st_global_16(row + half + 8 * c, as_u32x4(nhi));
  }
}

}  // namespace

hipError_t launch_rope(void *x, const int32_t *positions, int S, int H, int D, float base,
                       hipStream_t stream) {
  if (S <= 0 || H <= 0) return hipSuccess;
  const int chunks = D / 16;
  int tok = 512 / (H * chunks);
  if (tok < 1) tok = 1;
  if (tok > 64) tok = 64;
  while (tok > 1 && tok * (D / 2) > MAX_TABLE) --tok;
  dim3 grid((S + tok - 1) / tok), block(NT);
  hipLaunchKernelGGL(rope_kernel, grid, block, 0, stream, static_cast<bf16 *>(x), positions, S, H,
                     D, log2((double)base), tok);
  return hipGetLastError();
}

}  // namespace lcat

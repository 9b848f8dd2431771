// Rotary position embedding at absolute token positions, in place
// ("Ulysses sequence parallelism in long-context inference", §3.2 and §5.3;
// the angle arithmetic and its precision are described in rope_math.h).
//
// A workgroup handles a few consecutive tokens: it first builds the
// (cos, sin) table of those tokens in LDS (each angle once, shared by all
// heads), then streams the heads with 16-byte loads and stores.
#include "device.h"
#include "kernels.h"
#include "rope_math.h"

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

  for (int idx = tid; idx < nt * half; idx += NT) {
    const int t = idx / half, i = idx % half;
    cs[idx] = rope_cos_sin(rope_theta(i, D, log2_base), positions[t0 + t]);
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
    rope_rotate8(lo, hi, &cs[t * half + 8 * c], nlo, nhi);
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

// Rotary position embedding at absolute token positions, in place
// ("Ulysses sequence parallelism in long-context inference", §3.2 and §5.3;
// the angle arithmetic and its precision are described in rope_math.h).
//
// A workgroup handles a few consecutive tokens: it builds theta once and the
// (cos, sin) table of those tokens in LDS (each angle once, shared by all
// heads), then streams the heads with non-temporal 16-byte loads and
// stores.  Many small workgroups stream HBM faster here than fewer ones that
// each walk several token groups with their next loads issued ahead.
#include "device.h"
#include "kernels.h"
#include "rope_math.h"

namespace lcat {
namespace {

constexpr int NT = 128;
constexpr int UPT = 2;            // items per thread and batch
constexpr int MAX_TABLE = 4096;   // (token, frequency) pairs per workgroup

// Dynamic LDS: theta_i for i < D/2 (doubles), then the (cos, sin) table of
// the workgroup's tokens.  The first batch of loads is issued before the
// table is built, so its latency is hidden behind that arithmetic.
// Two tensors can be rotated in one launch (Q and K at the same positions):
// head h < H of a token is row h of x, head H + h2 is row h2 of x2, and the
// token's (cos, sin) table serves both.
__global__ __launch_bounds__(NT) void rope_kernel(bf16 *__restrict__ x, int H, bf16 *__restrict__ x2,
                                                  int H2, const int32_t *__restrict__ positions,
                                                  int S, int D, double log2_base, int tok_per_wg) {
  extern __shared__ __attribute__((aligned(16))) char rope_lds[];
  const int half = D >> 1;
  double *theta = reinterpret_cast<double *>(rope_lds);
  float2 *cs = reinterpret_cast<float2 *>(rope_lds + half * sizeof(double));
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * tok_per_wg;
  const int nt = min(tok_per_wg, S - t0);
  if (nt <= 0) return;

  const int chunks = half >> 3;                      // 8-element chunks per half
  const int Ht = H + H2;
  const int items = nt * Ht * chunks;
  bf16x8 lo[UPT], hi[UPT];
  auto row_of = [&](int it, int &c, int &t) __attribute__((always_inline)) -> bf16 * {
    c = it % chunks;
    const int th = it / chunks;
    const int h = th % Ht;
    t = th / Ht;
    return h < H ? x + ((size_t)(t0 + t) * H + h) * D : x2 + ((size_t)(t0 + t) * H2 + (h - H)) * D;
  };
  auto load = [&](int base) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int it = base + tid + u * NT;
      if (it < items) {
        int c, t;
        const bf16 *row = row_of(it, c, t);
        lo[u] = as_bf16x8(ld_global_16_nt(row + 8 * c));
        hi[u] = as_bf16x8(ld_global_16_nt(row + half + 8 * c));
      }
    }
  };
  load(0);

  for (int i = tid; i < half; i += NT) theta[i] = rope_theta(i, D, log2_base);
  __syncthreads();
  for (int idx = tid; idx < nt * half; idx += NT)
    cs[idx] = rope_cos_sin(theta[idx % half], positions[t0 + idx / half]);
  __syncthreads();

  for (int base = 0; base < items; base += NT * UPT) {
    if (base > 0) load(base);
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int it = base + tid + u * NT;
      if (it < items) {
        int c, t;
        bf16 *row = row_of(it, c, t);
        bf16x8 nlo, nhi;
        rope_rotate8(lo[u], hi[u], &cs[t * half + 8 * c], nlo, nhi);
        __builtin_nontemporal_store(as_u32x4(nlo), reinterpret_cast<u32x4 *>(row + 8 * c));
        __builtin_nontemporal_store(as_u32x4(nhi), reinterpret_cast<u32x4 *>(row + half + 8 * c));
      }
    }
  }
}

}  // namespace

hipError_t launch_rope(void *x, int H, void *x2, int H2, const int32_t *positions, int S, int D,
                       float base, hipStream_t stream) {
  if (S <= 0 || H + H2 <= 0) return hipSuccess;
  const int chunks = D / 16;
  int tok = NT * UPT / ((H + H2) * chunks);
  if (tok < 1) tok = 1;
  if (tok > 64) tok = 64;
  while (tok > 1 && tok * (D / 2) > MAX_TABLE) --tok;
  const size_t lds = (size_t)(D / 2) * sizeof(double) + (size_t)tok * (D / 2) * sizeof(float2);
  dim3 grid((S + tok - 1) / tok), block(NT);
  hipLaunchKernelGGL(rope_kernel, grid, block, lds, stream, static_cast<bf16 *>(x), H,
                     static_cast<bf16 *>(x2), H2, positions, S, D, log2((double)base), tok);
  return hipGetLastError();
}

}  // namespace lcat

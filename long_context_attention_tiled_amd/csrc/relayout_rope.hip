// Sequence-shard -> head-shard relayout of one rank's Q, K and V with RoPE
// applied to Q and K on the way, in one pass over HBM.
//
// "Ulysses sequence parallelism in long-context inference": §2.2 defines the
// relayout (after the exchange a GPU holds the complete sequence for its own
// heads), §3.2 binds every token to its absolute position through the global
// token index table and generates RoPE from it.  RoPE acts on each token's
// head rows independently, so it commutes with the relayout; doing both in
// one kernel moves Q and K once instead of twice (read + write of the
// relayout, then read + write of the in-place rotation).
//
// Work unit: one "pair" = chunk c (8 elements) of the first half of a head
// row together with chunk c of the second half, i.e. the eight rotate-half
// pairs (x[8c+e], x[D/2+8c+e]).  Consecutive threads take consecutive
// pairs (c fastest, then head, then token), so each wave reads and writes
// whole head rows.  A workgroup covers NT*UPT consecutive pairs of one
// tensor; for Q and K it first builds the (cos, sin) table of the tokens it
// touches in LDS (each frequency and each angle once, shared by its heads;
// the loads are issued before the table is built), with the arithmetic
// of rope_math.h so results match the in-place RoPE kernel bit for bit.  V
// takes the same path without the rotation.  Stores are non-temporal.
#include <algorithm>

#include "device.h"
#include "kernels.h"
#include "rope_math.h"

namespace lcat {
namespace {

constexpr int NT = 256;
constexpr int UPT = 2;   // pairs per thread (four 16-byte loads in flight)

struct RopeJob {
  const char *in;        // [SP][S_loc][H_tot][D] bf16
  char *out;             // [SP*S_loc][H_loc][D] bf16
  long long n_pairs;     // SP*S_loc*H_loc*hc
  long long wg_begin;    // first workgroup of this job in the launch
  int H_tot, H_loc, rank;
  int rotate;            // 1: Q or K (rotate), 0: V (copy)
};

// Dynamic LDS: theta_i for i < D/2 (doubles), then the (cos, sin) table,
// sized by the launch for the largest table any workgroup builds (a smaller
// table leaves room for more resident workgroups).
__global__ __launch_bounds__(NT) void permute_rope_kernel(RopeJob j0, RopeJob j1, RopeJob j2,
                                                          const int32_t *__restrict__ positions,
                                                          int D, double log2_base) {
  extern __shared__ __attribute__((aligned(16))) char rope_lds[];
  double *theta = reinterpret_cast<double *>(rope_lds);
  float2 *cs = reinterpret_cast<float2 *>(rope_lds + (D >> 1) * sizeof(double));
  const long long wg = blockIdx.x;
  const RopeJob &j = wg >= j2.wg_begin ? j2 : (wg >= j1.wg_begin ? j1 : j0);
  const int tid = threadIdx.x;
  const int half = D >> 1;
  const int hc = half >> 3;                       // chunks per half row
  const int per_tok = j.H_loc * hc;               // pairs per token
  const long long p0 = (wg - j.wg_begin) * (NT * UPT);
  const long long p_end = min(p0 + NT * UPT, j.n_pairs);
  const long long t_first = p0 / per_tok;
  const bool rot = j.rotate != 0;                 // uniform over the workgroup

  // loads first: they do not depend on the table, so their latency is
  // hidden behind its construction
  const long long row_bytes = 2LL * D;
  u32x4 lo[UPT], hi[UPT];
  long long dst[UPT];
  int tab[UPT];
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const long long p = p0 + tid + (long long)u * NT;
    const long long t = p / per_tok;
    const int rem = (int)(p - t * per_tok);
    const int h = rem / hc, c = rem - h * hc;
    const long long src = (t * j.H_tot + (long long)j.rank * j.H_loc + h) * row_bytes + 16LL * c;
    dst[u] = (t * j.H_loc + h) * row_bytes + 16LL * c;
    tab[u] = (int)(t - t_first) * half + 8 * c;
    if (p < p_end) {
      lo[u] = ld_global_16_nt(j.in + src);
      hi[u] = ld_global_16_nt(j.in + src + 2 * half);
    }
  }
  if (rot) {
    for (int i = tid; i < half; i += NT) theta[i] = rope_theta(i, D, log2_base);
    __syncthreads();
    const int n_tab = (int)((p_end - 1) / per_tok - t_first + 1) * half;
    for (int idx = tid; idx < n_tab; idx += NT) {
      const int t = idx / half, i = idx % half;
      cs[idx] = rope_cos_sin(theta[i], positions[t_first + t]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const long long p = p0 + tid + (long long)u * NT;
    if (p < p_end) {
      u32x4 a = lo[u], b = hi[u];
      if (rot) {
        bf16x8 nlo, nhi;
        rope_rotate8(as_bf16x8(a), as_bf16x8(b), &cs[tab[u]], nlo, nhi);
        a = as_u32x4(nlo);
        b = as_u32x4(nhi);
      }
      __builtin_nontemporal_store(a, reinterpret_cast<u32x4 *>(j.out + dst[u]));
      __builtin_nontemporal_store(b, reinterpret_cast<u32x4 *>(j.out + dst[u] + 2 * half));
    }
  }
}

}  // namespace

hipError_t launch_permute_qkv_rope(const void *const in[3], void *const out[3], const int H_tot[3],
                                   const int32_t *positions, int SP, int S_loc, int D, int rank,
                                   float base, hipStream_t stream) {
  const long long n_tok = (long long)SP * S_loc;
  if (n_tok == 0) return hipSuccess;
  const int hc = D / 16;
  RopeJob j[3];
  long long wg = 0;
  for (int t = 0; t < 3; ++t) {
    j[t].in = static_cast<const char *>(in[t]);
    j[t].out = static_cast<char *>(out[t]);
    j[t].H_tot = H_tot[t];
    j[t].H_loc = H_tot[t] / SP;
    j[t].rank = rank;
    j[t].rotate = t < 2;
    j[t].n_pairs = n_tok * j[t].H_loc * hc;
    j[t].wg_begin = wg;
    wg += (j[t].n_pairs + NT * UPT - 1) / (NT * UPT);
  }
  if (wg == 0) return hipSuccess;
  // Largest table: the NT*UPT pairs of a workgroup span at most
  // ceil(NT*UPT / pairs-per-token) + 1 tokens, each with D/2 frequencies.
  long long max_tab = 0;
  for (int t = 0; t < 2; ++t) {
    const long long per_tok = (long long)j[t].H_loc * hc;
    if (j[t].n_pairs > 0 && per_tok > 0)
      max_tab = std::max(max_tab, ((NT * UPT + per_tok - 1) / per_tok + 1) * (D / 2));
  }
  const size_t lds = (size_t)(D / 2) * sizeof(double) + (size_t)max_tab * sizeof(float2);
  if (lds > 64 * 1024) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(permute_rope_kernel, dim3((unsigned)wg), dim3(NT), lds, stream, j[0], j[1],
                     j[2], positions, D, log2((double)base));
  return hipGetLastError();
}

}  // namespace lcat

// Sequence-shard -> head-shard relayout of one rank.
//
// "Ulysses sequence parallelism in long-context inference", §2.2: after the
// first exchange each GPU holds the complete sequence for its own subset of
// heads (worked example: 4 shards of 16 tokens, 8 heads; GPU0 ends with heads
// 0 and 1 of all 64 tokens).  On one GPU the data movement of that step for
// rank r is the gather
//     out[k*S_loc + s][h][:] = in[k][s][r*H_loc + h][:]
// which is a batch of SP*S_loc contiguous runs of H_loc*D elements.  The
// copy is pure HBM traffic: each thread moves 16-byte units, several per
// thread with all loads issued before the stores, and consecutive threads
// take consecutive units so every wave reads and writes whole cache lines.
// Stores are non-temporal (streaming), which on gfx950 raises copy
// bandwidth from about 5.5 to about 7 TB/s.
#include "device.h"
#include "kernels.h"

namespace lcat {
namespace {

constexpr int NT = 256;
constexpr int UPT = 4;   // 16-byte units per thread

__global__ __launch_bounds__(NT) void permute16_kernel(const char *__restrict__ in,
                                                       char *__restrict__ out, long long n_units,
                                                       int units_per_run, int S_loc, int H_tot,
                                                       int H_loc, int rank, long long row_bytes) {
  const long long base = (long long)blockIdx.x * (NT * UPT) + threadIdx.x;
  u32x4 buf[UPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const long long u = base + (long long)i * NT;
    if (u < n_units) {
      const long long tok = u / units_per_run;
      const int w = (int)(u - tok * units_per_run);
      const long long src = (tok * H_tot + (long long)rank * H_loc) * row_bytes + 16LL * w;
      buf[i] = ld_global_16(in + src);
    }
  }
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const long long u = base + (long long)i * NT;
    // streaming store: the output is not read again by this kernel
    if (u < n_units) __builtin_nontemporal_store(buf[i], reinterpret_cast<u32x4 *>(out + 16LL * u));
  }
}

template <typename T>
__global__ __launch_bounds__(NT) void permute_elem_kernel(const T *__restrict__ in,
                                                          T *__restrict__ out, long long n_elem,
                                                          int run_elems, int H_tot, int H_loc,
                                                          int rank, int D) {
  const long long e = (long long)blockIdx.x * NT + threadIdx.x;
  if (e >= n_elem) return;
  const long long tok = e / run_elems;
  const int w = (int)(e - tok * run_elems);
  out[e] = in[(tok * H_tot + (long long)rank * H_loc) * D + w];
}

}  // namespace

hipError_t launch_permute(const void *in, void *out, int SP, int S_loc, int H_tot, int D, int rank,
                          int elem_bytes, hipStream_t stream) {
  const int H_loc = H_tot / SP;
  const long long n_tok = (long long)SP * S_loc;
  const long long run_bytes = (long long)H_loc * D * elem_bytes;
  if (n_tok == 0 || run_bytes == 0) return hipSuccess;
  const bool aligned16 = (reinterpret_cast<uintptr_t>(in) % 16 == 0) &&
                         (reinterpret_cast<uintptr_t>(out) % 16 == 0) && (run_bytes % 16 == 0) &&
                         (((long long)D * elem_bytes) % 16 == 0);
  if (aligned16) {
    const long long n_units = n_tok * (run_bytes / 16);
    const long long n_wg = (n_units + NT * UPT - 1) / (NT * UPT);
    hipLaunchKernelGGL(permute16_kernel, dim3((unsigned)n_wg), dim3(NT), 0, stream,
                       static_cast<const char *>(in), static_cast<char *>(out), n_units,
                       (int)(run_bytes / 16), S_loc, H_tot, H_loc, rank,
                       (long long)D * elem_bytes);
    return hipGetLastError();
  }
  const long long n_elem = n_tok * H_loc * D;
  const unsigned n_wg = (unsigned)((n_elem + NT - 1) / NT);
  const int run_elems = H_loc * D;
  switch (elem_bytes) {
    case 1:
      hipLaunchKernelGGL(permute_elem_kernel<uint8_t>, dim3(n_wg), dim3(NT), 0, stream,
                         static_cast<const uint8_t *>(in), static_cast<uint8_t *>(out), n_elem,
                         run_elems, H_tot, H_loc, rank, D);
      break;
    case 2:
      hipLaunchKernelGGL(permute_elem_kernel<uint16_t>, dim3(n_wg), dim3(NT), 0, stream,
                         static_cast<const uint16_t *>(in), static_cast<uint16_t *>(out), n_elem,
                         run_elems, H_tot, H_loc, rank, D);
      break;
    case 4:
      hipLaunchKernelGGL(permute_elem_kernel<uint32_t>, dim3(n_wg), dim3(NT), 0, stream,
                         static_cast<const uint32_t *>(in), static_cast<uint32_t *>(out), n_elem,
                         run_elems, H_tot, H_loc, rank, D);
      break;
    default:
      hipLaunchKernelGGL(permute_elem_kernel<uint64_t>, dim3(n_wg), dim3(NT), 0, stream,
                         static_cast<const uint64_t *>(in), static_cast<uint64_t *>(out), n_elem,
                         run_elems, H_tot, H_loc, rank, D);
      break;
  }
  return hipGetLastError();
}

}  // namespace lcat

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
// Loads and stores carry the non-temporal hint (streaming): with it the
// relayout of one rank's Q, K and V share at 64K moves 6.4 TB/s, against
// 5.9 TB/s with plain loads.
//
// The same kernel runs the reverse exchange of §2.2 (head shard back to
// sequence shards, each head at its global index as §2.3 asks): the
// contiguous side is then the input and the strided side the output,
//     out[k][s][r*H_loc + h][:] = in[k*S_loc + s][h][:]
#include "device.h"
#include "kernels.h"

namespace lcat {
namespace {

constexpr int NT = 256;
constexpr int UPT = 4;   // 16-byte units per thread

// One tensor's relayout in 16-byte units.  Unit u of the head-sharded
// (contiguous) side is unit (u mod units_per_run) of run (u div
// units_per_run), whose row on the sequence-sharded side is that token's
// first local head.  gather: strided in -> contiguous out; scatter: the
// reverse.
struct Permute16Job {
  const char *in;
  char *out;
  long long n_units;
  long long wg_begin;    // first workgroup of this job in the launch
  long long row_bytes;   // bytes of one head row (D * elem_bytes)
  int units_per_run;     // 16-byte units per token run (H_loc heads)
  int H_tot, H_loc, rank;
  int scatter;           // 0: sequence -> head shard, 1: head -> sequence shards
};

// Up to three jobs (Q, K, V) in one launch; each workgroup belongs to one job.
__global__ __launch_bounds__(NT) void permute16_kernel(Permute16Job j0, Permute16Job j1,
                                                       Permute16Job j2) {
  const long long wg = blockIdx.x;
  const Permute16Job &j = wg >= j2.wg_begin ? j2 : (wg >= j1.wg_begin ? j1 : j0);
  const long long base = (wg - j.wg_begin) * (NT * UPT) + threadIdx.x;
  u32x4 buf[UPT];
  long long strided[UPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const long long u = base + (long long)i * NT;
    const long long tok = u / j.units_per_run;
    const int w = (int)(u - tok * j.units_per_run);
    strided[i] = (tok * j.H_tot + (long long)j.rank * j.H_loc) * j.row_bytes + 16LL * w;
  }
  const bool sc = j.scatter != 0;   // uniform over the workgroup
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const long long u = base + (long long)i * NT;
    if (u < j.n_units) buf[i] = ld_global_16_nt(j.in + (sc ? 16LL * u : strided[i]));
  }
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const long long u = base + (long long)i * NT;
    // streaming store: the output is not read again by this kernel
    if (u < j.n_units)
      __builtin_nontemporal_store(buf[i],
                                  reinterpret_cast<u32x4 *>(j.out + (sc ? strided[i] : 16LL * u)));
  }
}

template <typename T>
__global__ __launch_bounds__(NT) void permute_elem_kernel(const T *__restrict__ in,
                                                          T *__restrict__ out, long long n_elem,
                                                          int run_elems, int H_tot, int H_loc,
                                                          int rank, int D, int scatter) {
  const long long e = (long long)blockIdx.x * NT + threadIdx.x;
  if (e >= n_elem) return;
  const long long tok = e / run_elems;
  const int w = (int)(e - tok * run_elems);
  const long long strided = (tok * H_tot + (long long)rank * H_loc) * D + w;
  if (scatter)
    out[strided] = in[e];
  else
    out[e] = in[strided];
}

}  // namespace

namespace {

bool fits16(const void *in, const void *out, int H_loc, int D, int elem_bytes) {
  const long long run_bytes = (long long)H_loc * D * elem_bytes;
  return (reinterpret_cast<uintptr_t>(in) % 16 == 0) && (reinterpret_cast<uintptr_t>(out) % 16 == 0) &&
         (run_bytes % 16 == 0) && (((long long)D * elem_bytes) % 16 == 0);
}

Permute16Job make_job(const void *in, void *out, long long n_tok, int H_tot, int SP, int D,
                      int rank, int elem_bytes, long long wg_begin, int scatter = 0) {
  Permute16Job j{};
  j.scatter = scatter;
  j.in = static_cast<const char *>(in);
  j.out = static_cast<char *>(out);
  j.H_tot = H_tot;
  j.H_loc = H_tot / SP;
  j.rank = rank;
  j.row_bytes = (long long)D * elem_bytes;
  j.units_per_run = (int)((long long)j.H_loc * D * elem_bytes / 16);
  j.n_units = n_tok * j.units_per_run;
  j.wg_begin = wg_begin;
  return j;
}

long long job_wgs(const Permute16Job &j) { return (j.n_units + NT * UPT - 1) / (NT * UPT); }

hipError_t launch_elem(const void *in, void *out, long long n_tok, int H_tot, int H_loc, int D,
                       int rank, int elem_bytes, int scatter, hipStream_t stream) {
  const long long n_elem = n_tok * H_loc * D;
  const unsigned n_wg = (unsigned)((n_elem + NT - 1) / NT);
  const int run_elems = H_loc * D;
  switch (elem_bytes) {
    case 1:
      hipLaunchKernelGGL(permute_elem_kernel<uint8_t>, dim3(n_wg), dim3(NT), 0, stream,
                         static_cast<const uint8_t *>(in), static_cast<uint8_t *>(out), n_elem,
                         run_elems, H_tot, H_loc, rank, D, scatter);
      break;
    case 2:
      hipLaunchKernelGGL(permute_elem_kernel<uint16_t>, dim3(n_wg), dim3(NT), 0, stream,
                         static_cast<const uint16_t *>(in), static_cast<uint16_t *>(out), n_elem,
                         run_elems, H_tot, H_loc, rank, D, scatter);
      break;
    case 4:
      hipLaunchKernelGGL(permute_elem_kernel<uint32_t>, dim3(n_wg), dim3(NT), 0, stream,
                         static_cast<const uint32_t *>(in), static_cast<uint32_t *>(out), n_elem,
                         run_elems, H_tot, H_loc, rank, D, scatter);
      break;
    default:
      hipLaunchKernelGGL(permute_elem_kernel<uint64_t>, dim3(n_wg), dim3(NT), 0, stream,
                         static_cast<const uint64_t *>(in), static_cast<uint64_t *>(out), n_elem,
                         run_elems, H_tot, H_loc, rank, D, scatter);
      break;
  }
  return hipGetLastError();
}

}  // namespace

namespace {

hipError_t launch_one(const void *in, void *out, int SP, int S_loc, int H_tot, int D, int rank,
                      int elem_bytes, int scatter, hipStream_t stream) {
  const int H_loc = H_tot / SP;
  const long long n_tok = (long long)SP * S_loc;
  if (n_tok == 0 || (long long)H_loc * D == 0) return hipSuccess;
  if (!fits16(in, out, H_loc, D, elem_bytes))
    return launch_elem(in, out, n_tok, H_tot, H_loc, D, rank, elem_bytes, scatter, stream);
  const Permute16Job j = make_job(in, out, n_tok, H_tot, SP, D, rank, elem_bytes, 0, scatter);
  const long long n_wg = job_wgs(j);
  Permute16Job none = j;
  none.wg_begin = n_wg;   // never selected
  hipLaunchKernelGGL(permute16_kernel, dim3((unsigned)n_wg), dim3(NT), 0, stream, j, none, none);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_permute(const void *in, void *out, int SP, int S_loc, int H_tot, int D, int rank,
                          int elem_bytes, hipStream_t stream) {
  return launch_one(in, out, SP, S_loc, H_tot, D, rank, elem_bytes, 0, stream);
}

hipError_t launch_unpermute(const void *in, void *out, int SP, int S_loc, int H_tot, int D,
                            int rank, int elem_bytes, hipStream_t stream) {
  return launch_one(in, out, SP, S_loc, H_tot, D, rank, elem_bytes, 1, stream);
}

hipError_t launch_permute_qkv(const void *const in[3], void *const out[3], const int H_tot[3],
                              int SP, int S_loc, int D, int rank, int elem_bytes,
                              hipStream_t stream) {
  const long long n_tok = (long long)SP * S_loc;
  if (n_tok == 0 || D == 0) return hipSuccess;
  bool all16 = true;
  for (int t = 0; t < 3; ++t) all16 = all16 && fits16(in[t], out[t], H_tot[t] / SP, D, elem_bytes);
  if (!all16) {
    for (int t = 0; t < 3; ++t) {
      const hipError_t e = launch_permute(in[t], out[t], SP, S_loc, H_tot[t], D, rank, elem_bytes,
                                          stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  Permute16Job j[3];
  long long wg = 0;
  for (int t = 0; t < 3; ++t) {
    j[t] = make_job(in[t], out[t], n_tok, H_tot[t], SP, D, rank, elem_bytes, wg);
    wg += job_wgs(j[t]);
  }
  if (wg == 0) return hipSuccess;
  hipLaunchKernelGGL(permute16_kernel, dim3((unsigned)wg), dim3(NT), 0, stream, j[0], j[1], j[2]);
  return hipGetLastError();
}

}  // namespace lcat

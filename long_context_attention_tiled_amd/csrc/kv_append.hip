// Append new tokens' K/V into the head-sharded paged cache.
//
// Layout ("Ulysses sequence parallelism in long-context inference", §2.3:
// KV kept per head in blocks of a separate pool, each block tagged with its
// global head index): a block holds 64 tokens of ONE KV head, K token-major
// [64][128] and V dimension-major [128][64] so attention kernels can feed V
// to the MFMA without a transpose.  Token -> slot follows the request-token
// to KV-slot map of the multi-GPU partitioning article, §2.1: position pos of
// request b goes to block block_table[b][g][pos/64], slot pos%64.
//
// One workgroup per (touched block, KV head, request).  K rows are copied
// with 16-byte vectors; V is transposed through LDS so that the pool writes
// are 128-byte coalesced rows.  Slots outside [start, start+T) are never
// written, so partially filled blocks keep their earlier tokens.
#include "device.h"
#include "kernels.h"

namespace lcat {
namespace {

constexpr int HD = 128;
constexpr int BT = 64;
constexpr int PITCH = HD + 2;   // bf16 elements per LDS row (odd word count: no bank conflicts)

__global__ __launch_bounds__(256) void kv_append_kernel(const bf16 *__restrict__ k_new,
                                                        const bf16 *__restrict__ v_new,
                                                        bf16 *__restrict__ k_pool,
                                                        bf16 *__restrict__ v_pool, int n_blocks,
                                                        const int32_t *__restrict__ block_head,
                                                        const int32_t *__restrict__ block_table,
                                                        int max_blocks,
                                                        const int32_t *__restrict__ start_pos,
                                                        int T, int Hkv, int kv_head_base,
                                                        int32_t *dev_status) {
  __shared__ uint16_t vt[BT * PITCH];
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

  // K: one 16-byte chunk per thread per step; V rows staged in LDS.
  for (int idx = tid; idx < BT * 16; idx += 256) {
    const int slot = idx >> 4, c = idx & 15;
    if (slot < s_lo || slot >= s_hi) continue;
    const int t = j * BT + slot - start;                // token index within the new tokens
    const size_t src = (((size_t)b * T + t) * Hkv + g) * HD + 8 * c;
    st_global_16(k_pool + ((size_t)blk * BT + slot) * HD + 8 * c, ld_global_16(k_new + src));
    const u32x4 vv = ld_global_16(v_new + src);
    uint32_t *row = reinterpret_cast<uint32_t *>(vt + slot * PITCH + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) row[e] = vv[e];
  }
  __syncthreads();
  // V^T: lane = slot, each wave walks a quarter of the channels.
  const int slot = tid & 63;
  if (slot >= s_lo && slot < s_hi) {
    uint16_t *dst = reinterpret_cast<uint16_t *>(v_pool) + (size_t)blk * HD * BT + slot;
    for (int d = tid >> 6; d < HD; d += 4) dst[(size_t)d * BT] = vt[slot * PITCH + d];
  }
}

}  // namespace

hipError_t launch_kv_append(const void *k_new, const void *v_new, void *k_pool, void *v_pool,
                            int n_blocks, const int32_t *block_head, const int32_t *block_table,
                            int max_blocks, const int32_t *start_pos, int T, int B, int Hkv,
                            int kv_head_base, int32_t *dev_status, hipStream_t stream) {
  if (T <= 0 || B <= 0) return hipSuccess;
  dim3 grid((T + BT - 1) / BT + 1, Hkv, B), block(256);
  hipLaunchKernelGGL(kv_append_kernel, grid, block, 0, stream, static_cast<const bf16 *>(k_new),
                     static_cast<const bf16 *>(v_new), static_cast<bf16 *>(k_pool),
                     static_cast<bf16 *>(v_pool), n_blocks, block_head, block_table, max_blocks,
                     start_pos, T, Hkv, kv_head_base, dev_status);
  return hipGetLastError();
}

}  // namespace lcat

// Tiled exact attention, bf16 MFMA on gfx950, head_dim 128.
//
// What is computed: softmax(scale * Q K^T) V with an optional causal mask on
// global token positions ("Flash Attention and distributed inference", §18.2
// for the result; §18.3 for the tiling: K/V tiles staged on chip, running
// row max m and denominator l, rescale of the output accumulator by
// exp(m_old - m_new) before adding each tile's P V; §18.4 for dividing by l
// once at the end and for putting the query tile in the outer loop so the
// grid runs over (query block, head, batch)).  The N x N score matrix never
// leaves registers.
//
// Mapping onto CDNA4:
//  * A workgroup is 8 waves.  All waves share one KV head: with a GQA group of
//    8 query heads each wave owns one query head and the same 32 query rows,
//    so one K/V tile in LDS feeds 8 x 32 query rows.  Smaller groups stack
//    query-row blocks instead; larger groups split over several workgroups.
//  * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys on
//    the M axis, its 32 queries on N).  In that layout a lane owns one query
//    and 32 keys of a 64-key tile, so the row max and row sum are lane-local
//    plus one exchange with lane l^32, and the rescale factor is one scalar
//    per lane.
//  * O^T = V^T P^T is the second MFMA: the exponentiated scores are already
//    in the B-operand layout once the K rows are read in a fixed permuted
//    order (bits 2 and 3 of the row swapped), so P never goes through LDS.
//    V is kept transposed in LDS (dimension-major) so its A-operand reads
//    are 16-byte vectors.
//  * The next K/V tile is fetched from HBM into registers while the current
//    tile is computed, then written to the other half of a double buffer.
//  * LDS rows are XOR-swizzled on 16-byte chunks so the MFMA operand reads
//    and the tile writes avoid bank conflicts.
#include "device.h"
#include "kernels.h"

namespace lcat {
namespace {

constexpr int HD = 128;                 // head dimension
constexpr int BN = 64;                  // keys per tile (= KV block)
constexpr int NW = 8;                   // waves per workgroup
constexpr int NT = NW * 64;             // threads per workgroup
constexpr int K_BYTES = BN * HD * 2;    // K tile   [64][128] bf16
constexpr int V_BYTES = HD * BN * 2;    // V^T tile [128][64] bf16
constexpr int STAGE = K_BYTES + V_BYTES;

__device__ __forceinline__ int k_lds_off(int row, int chunk) {
  return row * 256 + ((chunk ^ (row & 15)) << 4);
}

__device__ __forceinline__ int vt_lds_off(int d, int chunk) {
  return K_BYTES + d * 128 + ((chunk ^ (((d >> 1) ^ (d >> 3)) & 7)) << 4);
}

struct TileRegs {
  u32x4 r[4];
};

// Gather the 16-bit lane `i` (0..7) of four 8 x bf16 vectors into 4 x bf16.
__device__ __forceinline__ u32x2 column4(const TileRegs &t, int i) {
  const int w = i >> 1;
  u32x2 out;
  if (i & 1) {
    out.x = (t.r[0][w] >> 16) | (t.r[1][w] & 0xFFFF0000u);
    out.y = (t.r[2][w] >> 16) | (t.r[3][w] & 0xFFFF0000u);
  } else {
    out.x = (t.r[0][w] & 0xFFFFu) | (t.r[1][w] << 16);
    out.y = (t.r[2][w] & 0xFFFFu) | (t.r[3][w] << 16);
  }
  return out;
}

template <bool PAGED>
struct TileIO {
  // Issue the global loads of key tile `tile` into registers.
  //   threads   0..255 fetch V, threads 256..511 fetch K.
  // Keys at or past n_keys are never used in arithmetic: K rows there are
  // masked to -inf later, V entries are replaced by zeros here.
  static __device__ __forceinline__ void load(const PrefillParams &p, int b, int g, int tile,
                                              int n_keys, int tid, TileRegs &t) {
    const int key0 = tile * BN;
    const bf16 *kb = static_cast<const bf16 *>(p.k);
    const bf16 *vb = static_cast<const bf16 *>(p.v);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    if constexpr (PAGED) {
      const int blk = tile < p.max_blocks
                          ? p.block_table[((size_t)b * p.Hkv + g) * p.max_blocks + tile]
                          : -1;
      const bool ok = blk >= 0 && blk < p.n_blocks;
      if (tid == 0 && p.dev_status) {
        if (!ok)
          p.dev_status[0] = 2;
        else if (p.block_head[blk] != p.kv_head_base + g)
          p.dev_status[0] = 1;
      }
      const int nv = n_keys - key0;   // valid keys in this block (>= 1)
      if (tid < 256) {
        const int u = tid;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int d = 32 * pp + (u >> 3), c = u & 7;
          u32x4 x = ok ? ld_global_16(vb + ((size_t)blk * HD + d) * BN + 8 * c) : zero;
          if (nv < BN) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int k0 = 8 * c + 2 * e;
              uint32_t w = x[e];
              if (k0 >= nv) w &= 0xFFFF0000u;
              if (k0 + 1 >= nv) w &= 0x0000FFFFu;
              x[e] = w;
            }
          }
          t.r[pp] = x;
        }
      } else {
        const int u = tid - 256;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int row = 16 * pp + (u >> 4), c = u & 15;
          t.r[pp] = ok ? ld_global_16(kb + ((size_t)blk * BN + row) * HD + 8 * c) : zero;
        }
      }
    } else {
      if (tid < 256) {
        const int kq = tid >> 4, dc = tid & 15;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = key0 + 4 * kq + e;
          t.r[e] = key < n_keys
                       ? ld_global_16(vb + (((size_t)b * p.Sk + key) * p.Hkv + g) * HD + 8 * dc)
                       : zero;
        }
      } else {
        const int u = tid - 256;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int row = 16 * pp + (u >> 4), c = u & 15;
          const int key = key0 + row;
          t.r[pp] = key < n_keys
                        ? ld_global_16(kb + (((size_t)b * p.Sk + key) * p.Hkv + g) * HD + 8 * c)
                        : zero;
        }
      }
    }
  }

  // Write the fetched tile into one LDS stage (V transposed for dense input).
  static __device__ __forceinline__ void store(char *stage, int tid, const TileRegs &t) {
    if (tid < 256) {
      if constexpr (PAGED) {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int d = 32 * pp + (tid >> 3), c = tid & 7;
          *reinterpret_cast<u32x4 *>(stage + vt_lds_off(d, c)) = t.r[pp];
        }
      } else {
        const int kq = tid >> 4, dc = tid & 15;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int d = 8 * dc + i;
          *reinterpret_cast<u32x2 *>(stage + vt_lds_off(d, kq >> 1) + 8 * (kq & 1)) = column4(t, i);
        }
      }
    } else {
      const int u = tid - 256;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const int row = 16 * pp + (u >> 4), c = u & 15;
        *reinterpret_cast<u32x4 *>(stage + k_lds_off(row, c)) = t.r[pp];
      }
    }
  }
};

template <bool PAGED, bool CAUSAL>
__global__ __launch_bounds__(NT) void prefill_kernel(PrefillParams p, int heads_per_wg,
                                                     int head_slices, int n_qblk) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;   // query column of this lane within the wave's 32 rows
  const int gq = lane >> 5;   // which 8-wide half of each 16-long K slice

  // ---- workgroup -> (query block, batch, KV head, head slice) -------------
  const int per_q = p.B * p.Hkv * head_slices;
  int qblk = blockIdx.x / per_q;
  if (CAUSAL && !PAGED) qblk = n_qblk - 1 - qblk;   // longest rows first
  int rem = blockIdx.x % per_q;
  const int slice = rem % head_slices;
  rem /= head_slices;
  const int g = rem % p.Hkv;
  const int b = rem / p.Hkv;
  const int group = p.Hq / p.Hkv;
  const int h = g * group + slice * heads_per_wg + (wave % heads_per_wg);
  const int rows_wg = 32 * (NW / heads_per_wg);
  const int row0 = qblk * rows_wg + (wave / heads_per_wg) * 32;

  const int qoff = PAGED ? p.ctx_before[b] : 0;
  if (PAGED && (qoff < 0 || (long long)qoff + p.Sq > (long long)p.max_blocks * BN)) {
    // cached length outside what the block table can hold: flag, write nothing
    if (tid == 0 && p.dev_status) p.dev_status[0] = 2;
    return;
  }
  const int n_keys = PAGED ? qoff + p.Sq : p.Sk;
  int wave_keys = n_keys, wg_keys = n_keys;
  if (CAUSAL) {
    wave_keys = min(n_keys, qoff + min(row0 + 31, p.Sq - 1) + 1);
    wg_keys = min(n_keys, qoff + min(qblk * rows_wg + rows_wg - 1, p.Sq - 1) + 1);
  }
  if (row0 >= p.Sq) wave_keys = 0;
  const int n_tiles = (wg_keys + BN - 1) / BN;
  const int wave_tiles = (wave_keys + BN - 1) / BN;

  // ---- this wave's 32 query rows, held as the B operand of S^T = K Q^T ----
  const bf16 *qp = static_cast<const bf16 *>(p.q);
  const int qrow = row0 + lr;
  bf16x8 qf[8];
  {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bf16 *src = qp + (((size_t)b * p.Sq + qrow) * p.Hq + h) * HD + 8 * gq;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(qrow < p.Sq ? ld_global_16(src + 16 * s) : zero);
  }

  // K row read by this lane for S^T rows 0..31 (bits 2 and 3 swapped) so that
  // the score registers land directly in the B-operand order of P V.
  const int krow = (lr & ~12) | ((lr & 4) << 1) | ((lr & 8) >> 1);
  const float c2 = p.scale * kLog2e;
  const int qpos = qoff + qrow;

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  TileRegs tr;
  if (n_tiles > 0) {
    TileIO<PAGED>::load(p, b, g, 0, n_keys, tid, tr);
    TileIO<PAGED>::store(smem, tid, tr);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const char *cur = smem + (j & 1) * STAGE;
    if (j + 1 < n_tiles) TileIO<PAGED>::load(p, b, g, j + 1, n_keys, tid, tr);

    if (j < wave_tiles) {
      // ---- S^T = K Q^T over the 64-key tile (two 32-key halves) ----------
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(cur + k_lds_off(krow, 2 * s + gq));
        const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(cur + k_lds_off(krow + 32, 2 * s + gq));
        s0 = mfma_32x32x16(a0, qf[s], s0);
        s1 = mfma_32x32x16(a1, qf[s], s1);
      }

      // ---- mask: keys past the end, and (causal) keys after the query ----
      const int key0 = j * BN;
      const bool need_mask = (key0 + BN > n_keys) || (CAUSAL && key0 + BN - 1 > qoff + row0);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = key0 + 16 * (r >> 3) + 8 * gq + (r & 7);
          if (kk >= n_keys || (CAUSAL && kk > qpos)) s0[r] = -INFINITY;
          if (kk + 32 >= n_keys || (CAUSAL && kk + 32 > qpos)) s1[r] = -INFINITY;
        }
      }

      // ---- online softmax statistics (lane-local + one exchange) ---------
      float mx = s0[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s0[r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
      mx = fmaxf(mx, wave_shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float msc = (m_new == -INFINITY) ? 0.f : m_new * c2;
      const float alpha = fast_exp2(m_run * c2 - msc);
      m_run = m_new;

      bf16x8 pb[4];
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p0 = fast_exp2(s0[8 * u + e] * c2 - msc);
          const float p1 = fast_exp2(s1[8 * u + e] * c2 - msc);
          psum += p0 + p1;
          pb[u][e] = to_bf16(p0);
          pb[2 + u][e] = to_bf16(p1);
        }
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;

      // ---- O^T += V^T P^T ------------------------------------------------
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(cur + vt_lds_off(32 * db + lr, 2 * u + gq));
          acc[db] = mfma_32x32x16(a, pb[u], acc[db]);
        }
      }
    }

    if (j + 1 < n_tiles) TileIO<PAGED>::store(smem + ((j + 1) & 1) * STAGE, tid, tr);
    __syncthreads();
  }

  // ---- epilogue: divide by l once, store O (bf16) and LSE ----------------
  const float l_tot = l_run + wave_shfl_xor(l_run, 32);
  if (qrow < p.Sq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16 *op = static_cast<bf16 *>(p.o) + (((size_t)b * p.Sq + qrow) * p.Hq + h) * HD;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = to_bf16(acc[db][4 * rq + e] * inv);
        *reinterpret_cast<bf16x4 *>(op + 32 * db + 8 * rq + 4 * gq) = w;
      }
    }
    if (p.lse && gq == 0)
      p.lse[((size_t)b * p.Hq + h) * p.Sq + qrow] =
          l_tot > 0.f ? (m_run * c2 + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillParams &p, bool paged, hipStream_t stream) {
  const int group = p.Hq / p.Hkv;
  const int heads_per_wg = group >= NW ? NW : group;
  const int head_slices = group >= NW ? group / NW : 1;
  const int rows_wg = 32 * (NW / heads_per_wg);
  const int n_qblk = (p.Sq + rows_wg - 1) / rows_wg;
  const long long n_wg = (long long)n_qblk * p.B * p.Hkv * head_slices;
  if (n_wg <= 0) return hipSuccess;
  if (n_wg > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)n_wg), block(NT);
  const bool causal = p.causal != 0;
  if (paged) {
    hipLaunchKernelGGL((prefill_kernel<true, true>), grid, block, 0, stream, p, heads_per_wg,
                       head_slices, n_qblk);
  } else if (causal) {
    hipLaunchKernelGGL((prefill_kernel<false, true>), grid, block, 0, stream, p, heads_per_wg,
                       head_slices, n_qblk);
  } else {
    hipLaunchKernelGGL((prefill_kernel<false, false>), grid, block, 0, stream, p, heads_per_wg,
                       head_slices, n_qblk);
  }
  return hipGetLastError();
}

}  // namespace lcat

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

// Online-softmax rescale threshold in log2 units.  The running maximum m is
// only raised when a tile's maximum exceeds it by more than this, so most
// tiles skip the O/l rescale.  Exponentials are then bounded by 2^8, which
// fp32 (accumulators) and bf16 (P) hold without loss of relative precision;
// the result is unchanged because O and l always share the same m.
constexpr float kRescaleLog2 = 8.0f;

template <int N>
struct Int {
  static constexpr int value = N;
};

struct TileRegs {
  u32x4 r[4];
  int ok;    // paged: block id was in range
  int nv;    // paged: valid keys in this block
  int tag;   // paged: global KV-head tag read from the block
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

// Global -> register -> LDS movement of one 64-key tile.  Waves 0-3 move V,
// waves 4-7 move K; `wave` is wave-uniform so the split is a scalar branch.
// load() only issues memory reads (nothing consumes them until store(), which
// runs after the current tile's math), so the fetch overlaps the compute.
// Dense keys past the end are clamped to the last key (finite data whose
// scores are masked to -inf, so their P is exactly 0); paged slots past the
// end are zeroed before they reach LDS because they may hold anything,
// including NaN.
template <bool PAGED>
struct TileIO {
  static __device__ __forceinline__ void load(const PrefillParams &p, int b, int g, int tile,
                                              int blk, int n_keys, int tid, int wave,
                                              TileRegs &t) {
    const int key0 = tile * BN;
    const bf16 *kb = static_cast<const bf16 *>(p.k);
    const bf16 *vb = static_cast<const bf16 *>(p.v);
    if constexpr (PAGED) {
      t.ok = blk >= 0 && blk < p.n_blocks;
      const int sblk = t.ok ? blk : 0;
      t.nv = n_keys - key0;
      t.tag = p.block_head[sblk];
      if (wave < 4) {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int d = 32 * pp + (tid >> 3), c = tid & 7;
          t.r[pp] = ld_global_16(vb + ((size_t)sblk * HD + d) * BN + 8 * c);
        }
      } else {
        const int u = tid - 256;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int row = 16 * pp + (u >> 4), c = u & 15;
          t.r[pp] = ld_global_16(kb + ((size_t)sblk * BN + row) * HD + 8 * c);
        }
      }
    } else {
      const int last = n_keys - 1;
      if (wave < 4) {
        const int kq = tid >> 4, dc = tid & 15;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = min(key0 + 4 * kq + e, last);
          t.r[e] = ld_global_16(vb + (((size_t)b * p.Sk + key) * p.Hkv + g) * HD + 8 * dc);
        }
      } else {
        const int u = tid - 256;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int key = min(key0 + 16 * pp + (u >> 4), last);
          t.r[pp] = ld_global_16(kb + (((size_t)b * p.Sk + key) * p.Hkv + g) * HD + 8 * (u & 15));
        }
      }
    }
  }

  static __device__ __forceinline__ void store(const PrefillParams &p, int g, char *stage,
                                               int tid, int wave, TileRegs &t) {
    if constexpr (PAGED) {
      if (tid == 0 && p.dev_status) {
        if (!t.ok)
          p.dev_status[0] = 2;
        else if (t.tag != p.kv_head_base + g)
          p.dev_status[0] = 1;
      }
      if (!t.ok) {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) t.r[pp] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (wave < 4) {
      if constexpr (PAGED) {
        if (t.nv < BN) {
          const int c = tid & 7;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k0 = 8 * c + 2 * e;
            const uint32_t keep =
                (k0 >= t.nv ? 0u : 0xFFFFu) | (k0 + 1 >= t.nv ? 0u : 0xFFFF0000u);
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) t.r[pp][e] &= keep;
          }
        }
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // Rows past the end read the last row (finite data) and are never stored.
  const int qrow = row0 + lr;
  bf16x8 qf[8];
  {
    const int qr = min(qrow, p.Sq - 1);
    const bf16 *src =
        static_cast<const bf16 *>(p.q) + (((size_t)b * p.Sq + qr) * p.Hq + h) * HD + 8 * gq;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(ld_global_16(src + 16 * s));
    // Consume Q here so its loads are complete before the tile loop; the
    // loop then never waits on the memory counter before its QK^T MFMAs.
#pragma unroll
    for (int s = 0; s < 8; ++s) asm volatile("" ::"v"(as_u32x4(qf[s])));
  }

  // LDS operand addresses (stage 0).  K rows are read in a fixed permuted
  // order (bits 2 and 3 of the row swapped) so that the score registers land
  // directly in the B-operand order of P V; rows 32..63 sit 8 KiB further.
  // V^T rows 32*db + lr: the swizzle of row d+32 is that of row d with chunk
  // bit 2 flipped, so one address per chunk pair serves all four d blocks.
  const int krow = (lr & ~12) | ((lr & 4) << 1) | ((lr & 8) >> 1);
  int ka[8], va[4];
#pragma unroll
  for (int s = 0; s < 8; ++s) ka[s] = k_lds_off(krow, 2 * s + gq);
#pragma unroll
  for (int u = 0; u < 4; ++u) va[u] = vt_lds_off(lr, 2 * u + gq);

  const float c2 = p.scale * kLog2e;   // scores -> log2 units
  const int qpos = qoff + qrow;

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  float m2 = -INFINITY;   // running max of this lane's row, log2 units
  float l_run = 0.f;      // lane-partial denominator (keys of this lane)

  auto compute = [&](auto stage_tag, int j) {
    constexpr int SOFF = decltype(stage_tag)::value * STAGE;
    // ---- S^T = K Q^T over the 64-key tile (two 32-key halves) ------------
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(smem + SOFF + ka[s]);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(smem + SOFF + 8192 + ka[s]);
      s0 = mfma_32x32x16(a0, qf[s], s0);
      s1 = mfma_32x32x16(a1, qf[s], s1);
    }

    // ---- mask: keys past the end, and (causal) keys after the query ------
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

    // ---- online softmax statistics (lane-local + one exchange) -----------
    float mx = fmaxf(s0[0], s0[1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s0[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    const float mx2 = mx * c2;
    const bool grow = mx2 > m2 + kRescaleLog2;
    if (__ballot(grow)) {
      const float m_new = grow ? mx2 : m2;
      const float alpha = grow ? fast_exp2(m2 - m_new) : 1.f;
      m2 = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;
    }
    const float msc = (m2 == -INFINITY) ? 0.f : m2;

    bf16x8 pb[4];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p0 = fast_exp2(fmaf(s0[8 * u + e], c2, -msc));
        const float p1 = fast_exp2(fmaf(s1[8 * u + e], c2, -msc));
        psum += p0 + p1;
        pb[u][e] = to_bf16(p0);
        pb[2 + u][e] = to_bf16(p1);
      }
    }
    l_run += psum;

    // ---- O^T += V^T P^T --------------------------------------------------
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(smem + SOFF + 4096 * db +
                                                           va[u ^ (2 * (db & 1))]);
        acc[db] = mfma_32x32x16(a, pb[u], acc[db]);
      }
    }
  };

  // Paged: physical block of a tile, read one tile ahead of its data so the
  // table lookup never stalls the data fetch.
  const int32_t *table = PAGED ? p.block_table + ((size_t)b * p.Hkv + g) * p.max_blocks : nullptr;
  auto block_of = [&](int tile) -> int {
    if constexpr (PAGED) return tile < p.max_blocks ? table[tile] : -1;
    return 0;
  };

  // The looked-up id stays in a vector register until the fetch that needs
  // it (one tile later); only then is it made wave-uniform, so the lookup's
  // latency is never waited on right after it is issued.
  auto uniform_block = [&](int v) -> int {
    asm volatile("" : "+v"(v));
    return __builtin_amdgcn_readfirstlane(v);
  };

  TileRegs tr;
  int blk_next = block_of(0);
  if (n_tiles > 0) {
    TileIO<PAGED>::load(p, b, g, 0, uniform_block(blk_next), n_keys, tid, wave, tr);
    blk_next = block_of(1);
    TileIO<PAGED>::store(p, g, smem, tid, wave, tr);
  }
  __syncthreads();

  // Two tiles per trip so each LDS stage offset is a compile-time constant.
  for (int j = 0; j < n_tiles; j += 2) {
    if (j + 1 < n_tiles) {
      TileIO<PAGED>::load(p, b, g, j + 1, uniform_block(blk_next), n_keys, tid, wave, tr);
      blk_next = block_of(j + 2);
    }
    if (j < wave_tiles) compute(Int<0>{}, j);
    if (j + 1 < n_tiles) TileIO<PAGED>::store(p, g, smem + STAGE, tid, wave, tr);
    __syncthreads();
    if (j + 1 >= n_tiles) break;
    if (j + 2 < n_tiles) {
      TileIO<PAGED>::load(p, b, g, j + 2, uniform_block(blk_next), n_keys, tid, wave, tr);
      blk_next = block_of(j + 3);
    }
    if (j + 1 < wave_tiles) compute(Int<1>{}, j + 1);
    if (j + 2 < n_tiles) TileIO<PAGED>::store(p, g, smem, tid, wave, tr);
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
          l_tot > 0.f ? (m2 + __log2f(l_tot)) * kLn2 : -INFINITY;
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

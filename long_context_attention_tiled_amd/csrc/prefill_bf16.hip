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
constexpr int TILE = BN * HD * 2;       // bytes of one K tile [64][128] or V^T tile [128][64]

// LDS: K slots 0/1 at [0, 2*TILE), V^T slots 0/1 at [2*TILE, 4*TILE).
// Rows are XOR-swizzled on 16-byte chunks so that MFMA operand reads (8
// rows, same chunk) and tile writes hit distinct banks.
__device__ __forceinline__ int k_lds_off(int row, int chunk) {
  return row * 256 + ((chunk ^ (row & 15)) << 4);
}

__device__ __forceinline__ int vt_lds_off(int d, int chunk) {
  return 2 * TILE + d * 128 + ((chunk ^ (((d >> 1) ^ (d >> 3)) & 7)) << 4);
}

// Scheduling shape of a GEMM phase (NREADS LDS operand reads feeding 16
// MFMAs): keep a few reads in flight ahead of the MFMA that consumes them
// instead of hoisting all of them, which would cost many extra registers.
template <int NREADS>
__device__ __forceinline__ void interleave_reads_with_mfma() {
  constexpr int per = NREADS / 16;   // reads issued per MFMA in steady state
  __builtin_amdgcn_sched_group_barrier(0x100, 4 * per, 0);
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, per, 0);   // next DS read(s)
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

constexpr int QROWS_BYTES = 32 * HD * 2;   // one wave's 32 query rows in LDS

// Online-softmax rescale threshold in log2 units.  The running maximum m is
// only raised when a tile's maximum exceeds it by more than this, so most
// tiles skip the O/l rescale.  Exponentials are then bounded by 2^8, which
// fp32 (accumulators) and bf16 (P) hold without loss of relative precision;
// the result is unchanged because O and l always share the same m.
constexpr float kRescaleLog2 = 8.0f;

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

// Global -> register -> LDS movement of one 64-key tile by one group of four
// waves (`gt` = thread index within the group, 0..255).  fetch_*() only issues
// memory reads; store_*() runs a half-step later, so the fetch overlaps
// compute.  Reads go through a buffer descriptor whose base is the tile's
// first row (wave-uniform) and whose extent stops at the end of the tensor,
// with per-lane byte offsets that are the same for every tile: rows past the
// end of the tensor read as zero, rows past the key count belong to other
// positions (finite data whose scores are masked to -inf, so their P is
// exactly 0).  Paged slots past the key count are zeroed before they reach
// LDS because they may hold anything, including NaN.
struct TileOffsets {
  int k[4];   // byte offsets of this thread's four K chunks within a tile
  int v[4];   // byte offsets of this thread's four V chunks within a tile
};

template <bool PAGED>
struct TileIO {
  static __device__ __forceinline__ TileOffsets offsets(const PrefillParams &p, int gt) {
    TileOffsets o;
    if constexpr (PAGED) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        o.k[pp] = (16 * pp + (gt >> 4)) * (HD * 2) + 16 * (gt & 15);   // [64][128] block
        o.v[pp] = (32 * pp + (gt >> 3)) * (BN * 2) + 16 * (gt & 7);    // [128][64] block
      }
    } else {
      const int rs = p.Hkv * HD * 2;   // bytes between consecutive keys
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        o.k[pp] = (16 * pp + (gt >> 4)) * rs + 16 * (gt & 15);
        o.v[pp] = (4 * (gt >> 4) + pp) * rs + 16 * (gt & 15);
      }
    }
    return o;
  }

  // Descriptor over the tile starting at key tile*64 of (b, g) (dense), or
  // over one 16 KiB block (paged).
  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const PrefillParams &p,
                                                                     const void *base, int b,
                                                                     int g, int tile, int blk) {
    if constexpr (PAGED) {
      return make_rsrc(static_cast<const bf16 *>(base) + (size_t)blk * TILE / 2, TILE);
    } else {
      const size_t first = (((size_t)b * p.Sk + (size_t)tile * BN) * p.Hkv + g) * HD;
      const size_t total = (size_t)p.B * p.Sk * p.Hkv * HD;
      const size_t bytes = (total - first) * 2;
      return make_rsrc(static_cast<const bf16 *>(base) + first,
                       bytes > 0x7FFFFFFFu ? 0x7FFFFFFF : (int)bytes);
    }
  }

  static __device__ __forceinline__ void fetch_k(const PrefillParams &p, const TileOffsets &o,
                                                 int b, int g, int tile, int blk, int gt,
                                                 TileRegs &t) {
    int sblk = 0;
    if constexpr (PAGED) {
      t.ok = blk >= 0 && blk < p.n_blocks;
      sblk = t.ok ? blk : 0;
      t.tag = p.block_head[sblk];
    }
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(p, p.k, b, g, tile, sblk);
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) t.r[pp] = buf_load_16(r, o.k[pp], 0);
  }

  static __device__ __forceinline__ void fetch_v(const PrefillParams &p, const TileOffsets &o,
                                                 int b, int g, int tile, int blk, int n_keys,
                                                 int gt, TileRegs &t) {
    int sblk = 0;
    if constexpr (PAGED) {
      t.ok = blk >= 0 && blk < p.n_blocks;
      sblk = t.ok ? blk : 0;
      t.nv = n_keys - tile * BN;
    }
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(p, p.v, b, g, tile, sblk);
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) t.r[pp] = buf_load_16(r, o.v[pp], 0);
  }

  static __device__ __forceinline__ void store_k(const PrefillParams &p, int g, char *slot, int gt_,
                                                 TileRegs &t) {
    const int gt = opaque(gt_);
    if constexpr (PAGED) {
      if (gt == 0 && p.dev_status) {
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
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const int row = 16 * pp + (gt >> 4), c = gt & 15;
      *reinterpret_cast<u32x4 *>(slot + k_lds_off(row, c)) = t.r[pp];
    }
  }

  // V^T slot: paged blocks are already dimension-major; dense tiles are
  // transposed here (4 keys x 8 channels per thread -> 8 rows of 4 keys).
  static __device__ __forceinline__ void store_v(char *slot_base, int gt_, TileRegs &t) {
    const int gt = opaque(gt_);
    if constexpr (PAGED) {
      if (!t.ok) {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) t.r[pp] = u32x4{0u, 0u, 0u, 0u};
      }
      if (t.nv < BN) {
        const int c = gt & 7;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k0 = 8 * c + 2 * e;
          const uint32_t keep = (k0 >= t.nv ? 0u : 0xFFFFu) | (k0 + 1 >= t.nv ? 0u : 0xFFFF0000u);
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) t.r[pp][e] &= keep;
        }
      }
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const int d = 32 * pp + (gt >> 3), c = gt & 7;
        *reinterpret_cast<u32x4 *>(slot_base + vt_lds_off(d, c)) = t.r[pp];
      }
    } else {
      const int kq = gt >> 4, dc = gt & 15;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int d = 8 * dc + i;
        *reinterpret_cast<u32x2 *>(slot_base + vt_lds_off(d, kq >> 1) + 8 * (kq & 1)) = column4(t, i);
      }
    }
  }
};

// Schedule ("ping-pong").  Waves 0-3 form group A and fetch K tiles, waves
// 4-7 form group B and fetch V tiles; each SIMD runs one wave of each group.
// A wave alternates two kinds of half-step, separated by workgroup barriers:
//   GEMM(j):    O^T += V_{j-1}^T P_{j-1}^T   and   S_j^T = K_j Q^T    (MFMA)
//   SOFTMAX(j): mask, running max, exponentials P_j, denominator      (VALU)
// Group B runs half a step behind group A, so in every half-step one wave
// of each SIMD feeds the matrix core while the other runs the softmax.
// Half-step 2j:   A: fetch K_{j+1}; GEMM(j)   B: store V_j; SOFTMAX(j-1)
// Half-step 2j+1: A: SOFTMAX(j); store K_{j+1} B: fetch V_{j+1}; GEMM(j)
// K_j lives in K slot j%2 and V_j in V slot j%2; every store lands in a
// slot whose previous tile was last read at least one barrier earlier.
template <bool PAGED, bool CAUSAL>
__global__ __launch_bounds__(NT) void prefill_kernel(PrefillParams p, int heads_per_wg,
                                                     int head_slices, int n_qblk) {
  // K slots, V^T slots, then each wave's 32 query rows (8 KiB per wave).
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE + NW * QROWS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool grp_a = wave < 4;
  const int gt = tid & 255;   // thread index within its group
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

  // ---- this wave's 32 query rows, staged in its own LDS region ----------
  // (swizzled like K) and read as the B operand of S^T = K Q^T during each
  // GEMM half-step.  Rows past the end copy the last row (finite data) and
  // are never stored.
  const int qrow = row0 + lr;
  char *const qs = smem + 4 * TILE + wave * QROWS_BYTES;
  {
    const int c = lane & 15;
    const bf16 *qp = static_cast<const bf16 *>(p.q);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (lane >> 4) + 4 * i;
      const int qr = min(row0 + r, p.Sq - 1);
      const u32x4 x = ld_global_16(qp + (((size_t)b * p.Sq + qr) * p.Hq + h) * HD + 8 * c);
      *reinterpret_cast<u32x4 *>(qs + k_lds_off(r, c)) = x;
    }
  }
  const int qbase = (int)(qs - smem) + lr * 256;
  const int qx = gq ^ (lr & 15);     // chunk 2s+gq of row lr sits at (2s ^ (qx & 14)) | (qx & 1)

  // LDS operand addresses (slot 0).  K rows are read in a fixed permuted
  // order (bits 2 and 3 of the row swapped) so that the score registers land
  // directly in the B-operand order of P V; rows 32..63 sit 8 KiB further.
  // V^T rows 32*db + lr: the swizzle of row d+32 is that of row d with chunk
  // bit 2 flipped, so one address per chunk pair serves all four d blocks.
  const int krow = (lr & ~12) | ((lr & 4) << 1) | ((lr & 8) >> 1);
  const int kbase = krow * 256;
  const int kx = gq ^ (krow & 15);   // chunk 2s+gq lands at (2s ^ (kx & 14)) | (kx & 1)
  int va[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) va[u] = vt_lds_off(lr, 2 * u + gq);

  const float c2 = p.scale * kLog2e;   // scores -> log2 units
  const int qpos = qoff + qrow;

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  f32x16 s0 = f32x16{}, s1 = f32x16{};
  bf16x8 pb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) pb[u] = bf16x8{};
  float m2 = -INFINITY;   // running max of this lane's row, log2 units
  float l_run = 0.f;      // lane-partial denominator (keys of this lane)

  // GEMM(j): P_{j-1} V_{j-1} into O, then S_j = K_j Q^T.
  auto gemm = [&](int j) __attribute__((always_inline)) {
    if (j >= 1 && j - 1 < wave_tiles) {
      const int vso = ((j - 1) & 1) * TILE;
      int vr[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) vr[u] = opaque(va[u]) + vso;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(smem + 4096 * db +
                                                             vr[u ^ (2 * (db & 1))]);
          acc[db] = mfma_32x32x16(a, pb[u], acc[db]);
        }
      }
      interleave_reads_with_mfma<16>();
    }
    __builtin_amdgcn_sched_barrier(0);   // P is dead before S is produced
    if (j < n_tiles && j < wave_tiles) {
      const int kso = (j & 1) * TILE;
      const int kb0 = opaque(kbase) + kso, kx0 = opaque(kx);
      const int qb0 = opaque(qbase), qx0 = opaque(qx);
      s0 = f32x16{};
      s1 = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int ka = kb0 + ((2 * s) ^ kx0) * 16;
        const bf16x8 qf = *reinterpret_cast<const bf16x8 *>(smem + qb0 + ((2 * s) ^ qx0) * 16);
        const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(smem + ka);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(smem + 8192 + ka);
        s0 = mfma_32x32x16(a0, qf, s0);
        s1 = mfma_32x32x16(a1, qf, s1);
      }
      interleave_reads_with_mfma<24>();
    }
  };

  // SOFTMAX(j): mask S_j, update the running max (lazily), P_j and l.
  auto softmax = [&](int j) __attribute__((always_inline)) {
    if (j >= wave_tiles) return;
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
  };

  // Paged: physical block of a tile, read one tile ahead of its data.  The
  // id stays in a vector register until the fetch that needs it; only then is
  // it made wave-uniform, so the lookup latency is never waited on early.
  const int32_t *table =
      PAGED ? p.block_table + ((size_t)b * p.Hkv + g) * p.max_blocks : nullptr;
  auto block_of = [&](int tile) __attribute__((always_inline)) -> int {
    if constexpr (PAGED) return tile < p.max_blocks ? table[tile] : -1;
    return 0;
  };
  auto uniform_block = [&](int v) __attribute__((always_inline)) -> int {
    asm volatile("" : "+v"(v));
    return __builtin_amdgcn_readfirstlane(v);
  };

  // Each group runs its own copy of the loop (so each keeps only its own
  // loop-invariant addresses live).  One trip is GEMM(j) then SOFTMAX(j), so
  // S and the prefetched tile never cross the loop back-edge.  Group B starts
  // one half-step later (storing V_0), and both groups execute exactly
  // 2*n_tiles + 3 barriers, so the workgroup stays in step.
  auto run_group = [&](auto is_a_tag) __attribute__((always_inline)) {
    constexpr bool IS_A = decltype(is_a_tag)::value != 0;
    TileRegs tr;
    const TileOffsets to = TileIO<PAGED>::offsets(p, gt);
    int blk_next = block_of(0);
    if (n_tiles > 0) {
      if constexpr (IS_A) {
        TileIO<PAGED>::fetch_k(p, to, b, g, 0, uniform_block(blk_next), gt, tr);
        TileIO<PAGED>::store_k(p, g, smem, gt, tr);
      } else {
        TileIO<PAGED>::fetch_v(p, to, b, g, 0, uniform_block(blk_next), n_keys, gt, tr);
      }
      blk_next = block_of(1);
    }
    __syncthreads();
    if constexpr (!IS_A) {
      if (n_tiles > 0) TileIO<PAGED>::store_v(smem, gt, tr);   // V slot 0
      __syncthreads();
    }
#pragma clang loop unroll(disable)
    for (int j = 0; j <= n_tiles; ++j) {
      // GEMM half-step: issue the next tile's fetch, then P_{j-1}V_{j-1}, S_j.
      if (j + 1 < n_tiles) {
        if constexpr (IS_A)
          TileIO<PAGED>::fetch_k(p, to, b, g, j + 1, uniform_block(blk_next), gt, tr);
        else
          TileIO<PAGED>::fetch_v(p, to, b, g, j + 1, uniform_block(blk_next), n_keys, gt, tr);
        blk_next = block_of(j + 2);
      }
      gemm(j);
      __syncthreads();
      if (IS_A || j < n_tiles) {
        // SOFTMAX half-step: P_j from S_j, then publish the fetched tile.
        if (j < n_tiles) softmax(j);
        if (j + 1 < n_tiles) {
          if constexpr (IS_A)
            TileIO<PAGED>::store_k(p, g, smem + ((j + 1) & 1) * TILE, gt, tr);
          else
            TileIO<PAGED>::store_v(smem + ((j + 1) & 1) * TILE, gt, tr);
        }
        __syncthreads();
      }
    }
  };
  if (grp_a)
    run_group(Int<1>{});
  else
    run_group(Int<0>{});

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

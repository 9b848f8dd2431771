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
//    Each wave keeps its 32 query rows in registers for the whole kernel.
//  * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys on
//    the M axis, its 32 queries on N).  In that layout a lane owns one query
//    and 32 keys of a 64-key tile, so the row max and row sum are lane-local
//    plus one exchange with lane l^32, and the rescale factor is one scalar
//    per lane.
//  * O^T = V^T P^T is the second MFMA: the exponentiated scores are already
//    in the B-operand layout once the K rows are read in a fixed permuted
//    order (bits 2 and 3 of the row swapped), so P never goes through LDS.
//    The V^T operand is read from a key-major V tile with the transposing LDS
//    read (ds_read_b64_tr_b16); paged V blocks are stored dimension-major
//    and read directly.
//  * K and V tiles move from HBM to LDS by buffer loads that write LDS
//    directly (no register staging), into a ring of four slots per tensor,
//    two tiles ahead of the tile being computed.
//  * LDS rows are XOR-swizzled on 16-byte chunks so that MFMA operand reads
//    hit distinct banks; the swizzle is applied by choosing which global
//    chunk each lane of a DMA fetches.
#include "device.h"
#include "kernels.h"

namespace lcat {
namespace {

constexpr int HD = 128;                 // head dimension
constexpr int BN = 64;                  // keys per tile (= KV block)
constexpr int NW = 8;                   // waves per workgroup
constexpr int NT = NW * 64;             // threads per workgroup
constexpr int TILE = BN * HD * 2;       // bytes of one K tile [64][128] or V tile
constexpr int NSLOT = 4;                // ring slots per tensor
constexpr int AHEAD = 2;                // tiles in flight ahead of the one computed
constexpr int VBASE = NSLOT * TILE;     // V slots follow the K slots
constexpr int DMA_PER_TILE = TILE / 1024 / 4;   // 1 KiB DMA instructions per wave per tile
constexpr int NPRE = 8;                 // P V operands read before the barrier
static_assert(AHEAD + 2 <= NSLOT, "a slot is refilled only after both groups finished with it");
static_assert(DMA_PER_TILE == 4, "vmcnt waits below assume 4 DMA instructions per tile");

// K tile (and dense V tile): 64 key rows x 16 chunks of 8 dims (256 B rows).
// Chunk c of K row r sits at position c ^ (r & 15): the 16 rows read by one
// quarter-wave in the S = K Q^T operand read fall on distinct banks.
__device__ __forceinline__ int k_pos(int row, int c) { return c ^ (row & 15); }
// Dense V rows: chunk c of row r at c ^ 4*(r & 3).  A transposing read takes
// 4 consecutive rows x 64 bytes per half-wave; this spreads them over all banks.
__device__ __forceinline__ int vd_pos(int row, int c) { return c ^ ((row & 3) << 2); }
// Paged V^T tile (dimension-major, 128 rows x 8 chunks of 8 keys, 128 B rows).
__device__ __forceinline__ int vp_pos(int d, int c) { return c ^ (((d >> 1) ^ (d >> 3)) & 7); }

// Online-softmax rescale threshold in log2 units.  The running maximum m is
// only raised when a tile's maximum exceeds it by more than this, so most
// tiles skip the O/l rescale.  Exponentials are then bounded by 2^8, which
// fp32 (accumulators) and bf16 (P) hold without loss of relative precision;
// the result is unchanged because O and l always share the same m.
constexpr float kRescaleLog2 = 8.0f;

typedef __attribute__((address_space(4))) const int32_t const_i32;

// Zero the elements of an 8-key operand whose key index (key_first + e) is at
// or past nv.  Used only on the last tile of a paged sequence, whose slots
// past the key count may hold anything, including NaN.
__device__ __forceinline__ bf16x8 mask_keys(bf16x8 a, int key_first, int nv) {
  u32x4 w = as_u32x4(a);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int k = key_first + 2 * e;
    w[e] &= (k < nv ? 0x0000FFFFu : 0u) | (k + 1 < nv ? 0xFFFF0000u : 0u);
  }
  return as_bf16x8(w);
}

// Schedule ("ping-pong").  Waves 0-3 form group A and fetch K tiles, waves
// 4-7 form group B and fetch V tiles; each SIMD runs one wave of each group.
// A wave alternates two kinds of half-step, separated by workgroup barriers:
//   GEMM(j):    O^T += V_{j-1}^T P_{j-1}^T   and   S_j^T = K_j Q^T    (MFMA)
//   SOFTMAX(j): mask, running max, exponentials P_j, denominator      (VALU)
// Group B runs half a step behind group A, so in every half-step one wave
// of each SIMD feeds the matrix core while the other runs the softmax.
//   half-step 2j:   A: fetch K_{j+2}; GEMM(j)     B: SOFTMAX(j-1); V_j ready
//   half-step 2j+1: A: SOFTMAX(j); K_{j+1} ready  B: fetch V_{j+2}; GEMM(j)
// "ready" = the fetching waves wait for their DMA and the next barrier
// publishes the tile.  Tile t lives in slot t % 4 of its ring; a slot is
// refilled two half-steps after its last reader finished.  At the end of
// SOFTMAX(j) a wave already reads the first half of the V_j operands it
// needs in GEMM(j+1), so they arrive while it waits at the barrier.
template <bool PAGED, bool CAUSAL>
__global__ __launch_bounds__(NT) void prefill_kernel(PrefillParams p, int heads_per_wg,
                                                     int head_slices, int n_qblk) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * NSLOT * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool grp_a = wave < 4;
  const int w4 = wave & 3;    // wave index within its group
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

  // ---- this wave's 32 query rows -> registers (B operand of S^T = K Q^T) --
  // qf[s] = dims 16s + 8gq .. +7 of query row row0 + lr.  Rows past the end
  // repeat the last row (finite data) and are never stored.
  const int qrow = row0 + lr;
  bf16x8 qf[8];
  {
    const int qr = min(qrow, p.Sq - 1);
    const bf16 *qp = static_cast<const bf16 *>(p.q) + (((size_t)b * p.Sq + qr) * p.Hq + h) * HD;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(ld_global_16(qp + 16 * s + 8 * gq));
#pragma unroll
    for (int s = 0; s < 8; ++s) asm volatile("" ::"v"(qf[s]));   // wait for Q here, not in the loop
  }

  // LDS operand addresses.  K rows are read in a fixed permuted order (bits
  // 2 and 3 of the row swapped) so that the score registers land directly in
  // the B-operand order of P V; rows 32..63 sit 8 KiB further.
  const int krow = (lr & ~12) | ((lr & 4) << 1) | ((lr & 8) >> 1);
  const int kbase = krow * 256;
  const int kx = gq ^ (krow & 15);   // chunk 2s+gq lands at (2s ^ (kx & 14)) | (kx & 1)
  // V^T operand for (key step u, dim block db): dense tiles via transposing
  // reads (two 8-byte reads per operand, at +4096u and +4096u+1024), paged
  // V^T tiles via one 16-byte read of row 32db+lr.
  int va[4];
  if constexpr (PAGED) {
#pragma unroll
    for (int u = 0; u < 4; ++u) va[u] = lr * 128 + ((vp_pos(lr, 2 * u + gq)) << 4);
  } else {
    const int q4 = (lane >> 2) & 3;
    const int r0 = 8 * (lane >> 5) + q4;
    const int c0 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) va[db] = r0 * 256 + 16 * (4 * (db ^ q4) + c0) + 8 * (lane & 1);
  }
  auto read_v = [&](int vslot, int u, int db) __attribute__((always_inline)) -> bf16x8 {
    if constexpr (PAGED) {
      return *reinterpret_cast<const bf16x8 *>(smem + vslot + va[u ^ (2 * (db & 1))] + 4096 * db);
    } else {
      const char *a = smem + vslot + va[db] + 4096 * u;
      const u32x2 lo = lds_read_tr16(a), hi = lds_read_tr16(a + 1024);
      return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
    }
  };

  const float c2 = p.scale * kLog2e;   // scores -> log2 units
  const int qpos = qoff + qrow;

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  f32x16 s0 = f32x16{}, s1 = f32x16{};
  bf16x8 pb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) pb[u] = bf16x8{};
  bf16x8 vpre[NPRE];
#pragma unroll
  for (int i = 0; i < NPRE; ++i) vpre[i] = bf16x8{};
  float m2 = -INFINITY;   // running max of this lane's row, log2 units
  float l_run = 0.f;      // lane-partial denominator (keys of this lane)

  // GEMM(j): P_{j-1} V_{j-1} into O, then S_j = K_j Q^T.
  auto gemm = [&](int j) __attribute__((always_inline)) {
    if (j >= 1 && j - 1 < wave_tiles) {
      const int vslot = VBASE + ((j - 1) % NSLOT) * TILE;
      const int nv = n_keys - (j - 1) * BN;   // valid keys in this tile
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int i = 4 * u + db;
          bf16x8 a = i < NPRE ? vpre[i < NPRE ? i : 0] : read_v(vslot, u, db);
          if (PAGED && nv < BN) a = mask_keys(a, 16 * u + 8 * gq, nv);
          acc[db] = mfma_32x32x16(a, pb[u], acc[db]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // P is dead before S is produced
    if (j < n_tiles && j < wave_tiles) {
      const int kb0 = opaque(kbase) + (j % NSLOT) * TILE, kx0 = opaque(kx);
      s0 = f32x16{};
      s1 = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int ka = kb0 + ((2 * s) ^ kx0) * 16;
        const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(smem + ka);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(smem + 8192 + ka);
        s0 = mfma_32x32x16(a0, qf[s], s0);
        s1 = mfma_32x32x16(a1, qf[s], s1);
      }
    }
  };

  // SOFTMAX(j): mask S_j, update the running max (lazily), P_j and l.
  auto softmax = [&](int j) __attribute__((always_inline)) {
    const int key0 = j * BN;
    const bool need_mask = (key0 + BN > n_keys) || (CAUSAL && key0 + BN - 1 > qoff + row0);
    if (need_mask) {
      const int lim = CAUSAL ? min(n_keys - 1, qpos) : n_keys - 1;   // last visible key
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = key0 + 16 * (r >> 3) + 8 * gq + (r & 7);
        if (kk > lim) s0[r] = -INFINITY;
        if (kk + 32 > lim) s1[r] = -INFINITY;
      }
    }
    float mx = fmaxf(s0[0], s0[1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s0[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
    mx = pair_max32(mx);
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
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[u][e] = to_bf16(fast_exp2(fmaf(s0[8 * u + e], c2, -msc)));
        pb[2 + u][e] = to_bf16(fast_exp2(fmaf(s1[8 * u + e], c2, -msc)));
      }
    }
    // l accumulates the bf16-rounded P, i.e. exactly the weights P V uses.
    float psum = l_run;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 w = as_u32x4(pb[u]);
#pragma unroll
      for (int e = 0; e < 4; ++e) psum = add_bf16_pair(w[e], psum);
    }
    l_run = psum;
  };

  // First NPRE operands of P_j V_j, read while the wave waits at the barrier.
  auto prefetch_v = [&](int j) __attribute__((always_inline)) {
    const int vslot = VBASE + (j % NSLOT) * TILE;
#pragma unroll
    for (int i = 0; i < NPRE; ++i) vpre[i] = read_v(vslot, i / 4, i % 4);
  };

  // ---- tile fetch: this group's tensor, 4 DMA instructions per wave -------
  // Instruction i of wave w4 fills LDS bytes [(4*w4 + i) KiB, +1 KiB) of the
  // slot: key rows 16*w4 + 4i .. +3 (K, dense V) or dimension rows
  // 32*w4 + 8i .. +7 (paged V^T).  Each lane picks the global chunk whose
  // swizzled position is its own LDS position.
  const int32_t *table =
      PAGED ? p.block_table + ((size_t)b * p.Hkv + g) * p.max_blocks : nullptr;
  auto block_of = [&](int tile) __attribute__((always_inline)) -> int {
    if constexpr (PAGED) return tile < p.max_blocks ? ((const const_i32 *)table)[tile] : -1;
    return 0;
  };

  auto run_group = [&](auto is_a_tag) __attribute__((always_inline)) {
    constexpr bool IS_A = decltype(is_a_tag)::value != 0;
    constexpr bool KEY_MAJOR = IS_A || !PAGED;
    const int rs = PAGED ? HD * 2 : p.Hkv * HD * 2;   // bytes between key rows
    int voff[DMA_PER_TILE];
#pragma unroll
    for (int i = 0; i < DMA_PER_TILE; ++i) {
      if constexpr (KEY_MAJOR) {
        const int r = 16 * w4 + 4 * i + (lane >> 4), pos = lane & 15;
        voff[i] = r * rs + 16 * (IS_A ? k_pos(r, pos) : vd_pos(r, pos));
      } else {
        const int d = 32 * w4 + 8 * i + (lane >> 3), pos = lane & 7;
        voff[i] = d * (BN * 2) + 16 * vp_pos(d, pos);
      }
    }
    char *const ring = smem + (IS_A ? 0 : VBASE) + w4 * 4096;
    const bf16 *const src = static_cast<const bf16 *>(IS_A ? p.k : p.v);

    auto issue = [&](int tile, int blk) __attribute__((always_inline)) {
      u32x4 r;
      if constexpr (PAGED) {
        const bool ok = blk >= 0 && blk < p.n_blocks;
        r = rsrc_words(src + (size_t)(ok ? blk : 0) * (TILE / 2), ok ? TILE : 0);
        if (IS_A && w4 == 0 && lane == 0 && p.dev_status) {
          if (!ok)
            p.dev_status[0] = 2;
          else if (((const const_i32 *)p.block_head)[blk] != p.kv_head_base + g)
            p.dev_status[0] = 1;
        }
      } else {
        // the range ends at key row Sk of this batch: later rows read as zero
        const size_t first = (((size_t)b * p.Sk + (size_t)tile * BN) * p.Hkv + g) * HD;
        const long long bytes = ((long long)(p.Sk - tile * BN) * p.Hkv - g) * HD * 2;
        r = rsrc_words(src + first, bytes > 0x7FFFFFFFLL ? 0x7FFFFFFF : (int)bytes);
      }
      char *const dst = ring + (tile % NSLOT) * TILE;
#pragma unroll
      for (int i = 0; i < DMA_PER_TILE; ++i) dma_to_lds_16(r, dst + i * 1024, voff[i]);
    };
    // wait until tile t's DMA from this wave has landed (tiles issued later
    // may stay in flight)
    auto wait_tile = [&](int t) __attribute__((always_inline)) {
      if (t + 1 < n_tiles)
        wait_vmcnt<DMA_PER_TILE>();
      else
        wait_vmcnt<0>();
    };

    int blk_next = 0;
    if (n_tiles > 0) {
      issue(0, block_of(0));
      if (n_tiles > 1) issue(1, block_of(1));
      blk_next = block_of(AHEAD);
      wait_tile(0);
    }
    barrier_no_wait();
    if constexpr (!IS_A) barrier_no_wait();   // half-step 0: nothing to do yet
#pragma clang loop unroll(disable)
    for (int j = 0; j <= n_tiles; ++j) {
      // GEMM half-step
      if (j + AHEAD < n_tiles) {
        issue(j + AHEAD, blk_next);
        blk_next = block_of(j + AHEAD + 1);
      }
      gemm(j);
      barrier_no_wait();
      if (IS_A || j < n_tiles) {
        // SOFTMAX half-step; then make the next tile ready and pre-read the
        // first P V operands of this tile
        if (j < n_tiles) {
          if (j < wave_tiles) softmax(j);
          if (PAGED) asm volatile("" ::"s"(blk_next));   // block id lands here, not later
          wait_tile(j + 1);
          if (NPRE > 0 && j < wave_tiles) prefetch_v(j);
        }
        barrier_no_wait();
      }
    }
  };
  if (grp_a)
    run_group(Int<1>{});
  else
    run_group(Int<0>{});

  // ---- epilogue: divide by l once, store O (bf16) and LSE ----------------
  const float l_tot = pair_sum32(l_run);
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

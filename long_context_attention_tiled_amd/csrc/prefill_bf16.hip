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
constexpr int NKS = 4;                  // K ring slots
constexpr int NVS = 4;                  // V ring slots (after the K slots)
constexpr int KA = 4;                   // iteration j fetches K_{j+KA}
constexpr int VA = 2;                   // iteration j fetches V_{j+VA}
constexpr int NPV = 4;                  // P V operands read before the barrier
constexpr int NPK = 4;                  // K Q^T operands read before the barrier
// K_t is read (operands) from the end of iteration t-2 to iteration t-1 and
// refilled by K_{t+NKS} in iteration t+NKS-KA; V_t is read from the end of
// iteration t to iteration t+1 and refilled in iteration t+NVS-VA.
static_assert(NKS - KA >= 0 && NVS - VA >= 2, "a slot is refilled only after its last reader");
static_assert(TILE / 1024 == 2 * NW, "each wave moves two 1 KiB pieces of a tile");

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

// Schedule (software pipelined within each wave).  Iteration j of a wave
// interleaves three independent pieces of work in one instruction stream:
//   O^T += V_{j-1}^T P_{j-1}^T      (16 MFMA, operands from the V ring)
//   softmax of S_j -> P_j, m, l     (VALU: max, exp2, bf16 pack, row sum)
//   S_{j+1}^T = K_{j+1} Q^T         (16 MFMA, operands from the K ring)
// so the matrix core and the vector ALU of a SIMD are busy at the same time
// in each wave (a wave can issue about four VALU instructions between two
// back-to-back MFMAs for free).  All 8 waves run the same schedule and meet
// at one barrier per iteration.
// Tile movement: iteration j fetches K_{j+4} and V_{j+2} (each wave moves
// 2 KiB of each tile); at its end every wave waits for the DMAs it issued in
// iteration j-1, so after the barrier K_{j+3} and V_{j+1} are complete.
// Each ring has four slots; a slot is refilled one iteration after its last
// reader.  Before the barrier a wave already reads the first operands of
// the next iteration (V_j for P_j V_j and K_{j+2} for S_{j+2}).
// Tiles that need the causal/length mask, and the first and last
// iterations, take a plain sequential path instead of the interleaved one.
template <bool PAGED, bool CAUSAL>
__global__ __launch_bounds__(NT) void prefill_kernel(PrefillParams p, int heads_per_wg,
                                                     int head_slices, int n_qblk) {
  __shared__ __attribute__((aligned(1024))) char smem[(NKS + NVS) * TILE];

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

  // ---- LDS operand addresses (within a slot) ------------------------------
  // K rows are read in a fixed permuted order (bits 2 and 3 of the row
  // swapped) so that the score registers land directly in the B-operand
  // order of P V; rows 32..63 sit 8 KiB further.  K operand s (s = 0..7,
  // dims 16s .. 16s+15) of half hf is at kaddr[s] + 8192 hf.
  const int krow = (lr & ~12) | ((lr & 4) << 1) | ((lr & 8) >> 1);
  int kaddr[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) kaddr[s] = krow * 256 + (k_pos(krow, 2 * s + gq) << 4);
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
  // operand i = 4u + db of P V for the V tile in LDS slot `vs` (byte offset)
  auto read_v = [&](int vs, int i) __attribute__((always_inline)) -> bf16x8 {
    const int u = i >> 2, db = i & 3;
    if constexpr (PAGED) {
      return *reinterpret_cast<const bf16x8 *>(smem + vs + va[u ^ (2 * (db & 1))] + 4096 * db);
    } else {
      const char *a = smem + vs + va[db] + 4096 * u;
      const u32x2 lo = lds_read_tr16(a), hi = lds_read_tr16(a + 1024);
      return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
    }
  };
  // operand i = 2s + hf of S = K Q^T for the K tile in LDS slot `ks`
  auto read_k = [&](int ks, int i) __attribute__((always_inline)) -> bf16x8 {
    return *reinterpret_cast<const bf16x8 *>(smem + ks + kaddr[i >> 1] + 8192 * (i & 1));
  };
  auto kslot = [](int t) { return (t % NKS) * TILE; };
  auto vslot = [](int t) { return (NKS + t % NVS) * TILE; };

  const float c2 = p.scale * kLog2e;   // scores -> log2 units
  const int qpos = qoff + qrow;

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  f32x16 S[2][2];        // S[parity][half]: scores of tile j in S[j & 1]
  bf16x8 P[2][4];        // P[parity][u]:    probabilities of tile j in P[j & 1]
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    S[a][0] = S[a][1] = f32x16{};
#pragma unroll
    for (int u = 0; u < 4; ++u) P[a][u] = bf16x8{};
  }
  bf16x8 vpre[NPV], kpre[NPK];   // operands read before the barrier
#pragma unroll
  for (int i = 0; i < NPV; ++i) vpre[i] = bf16x8{};
#pragma unroll
  for (int i = 0; i < NPK; ++i) kpre[i] = bf16x8{};
  float m2 = -INFINITY;   // running max of this lane's row, log2 units
  float l_run = 0.f;      // lane-partial denominator (keys of this lane)

  // ---- plain (sequential) pieces, used for edge iterations ----------------
  auto pv_plain = [&](int t, const bf16x8 (&pp)[4]) __attribute__((always_inline)) {
    const int vs = vslot(t);
    const int nv = n_keys - t * BN;   // valid keys in this tile
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      bf16x8 a = i < NPV ? vpre[i < NPV ? i : 0] : read_v(vs, i);
      if (PAGED && nv < BN) a = mask_keys(a, 16 * (i >> 2) + 8 * gq, nv);
      acc[i & 3] = mfma_32x32x16(a, pp[i >> 2], acc[i & 3]);
    }
  };
  auto s_plain = [&](int t, f32x16 (&sn)[2], bool use_pre) __attribute__((always_inline)) {
    const int ks = kslot(t);
    sn[0] = sn[1] = f32x16{};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bf16x8 a = (i < NPK && use_pre) ? kpre[i < NPK ? i : 0] : read_k(ks, i);
      sn[i & 1] = mfma_32x32x16(a, qf[i >> 1], sn[i & 1]);
    }
  };
  // Row max of a score tile (tree of max3) and the lazily raised running max.
  auto tile_max = [&](const f32x16 (&sc)[2]) __attribute__((always_inline)) -> float {
    float t[11];
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      const int a = 3 * i, b2 = 3 * i + 1, c = 3 * i + 2;
      t[i] = fmaxf(fmaxf(sc[a >> 4][a & 15], sc[b2 >> 4][b2 & 15]), sc[c >> 4][c & 15]);
    }
    t[10] = fmaxf(sc[1][14], sc[1][15]);
    const float u0 = fmaxf(fmaxf(t[0], t[1]), t[2]), u1 = fmaxf(fmaxf(t[3], t[4]), t[5]);
    const float u2 = fmaxf(fmaxf(t[6], t[7]), t[8]), u3 = fmaxf(t[9], t[10]);
    return pair_max32(fmaxf(fmaxf(u0, u1), fmaxf(u2, u3)));
  };
  // exp2 of half hf of the scores into P (bf16), returning the partial row sum
  auto exp_half = [&](const f32x16 (&sc)[2], bf16x8 (&pc)[4], int hf, float msc,
                      float psum) __attribute__((always_inline)) -> float {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pc[2 * hf + u][e] = to_bf16(fast_exp2(fmaf(sc[hf][8 * u + e], c2, -msc)));
      const u32x4 w = as_u32x4(pc[2 * hf + u]);
#pragma unroll
      for (int e = 0; e < 4; ++e) psum = add_bf16_pair(w[e], psum);
    }
    return psum;
  };
  auto softmax_plain = [&](int t, f32x16 (&sc)[2], bf16x8 (&pc)[4]) __attribute__((always_inline)) {
    const int key0 = t * BN;
    const bool need_mask = (key0 + BN > n_keys) || (CAUSAL && key0 + BN - 1 > qoff + row0);
    if (need_mask) {
      const int lim = CAUSAL ? min(n_keys - 1, qpos) : n_keys - 1;   // last visible key
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = key0 + 16 * (r >> 3) + 8 * gq + (r & 7);
        if (kk > lim) sc[0][r] = -INFINITY;
        if (kk + 32 > lim) sc[1][r] = -INFINITY;
      }
    }
    const float mx2 = tile_max(sc) * c2;
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
    l_run = exp_half(sc, pc, 1, msc, exp_half(sc, pc, 0, msc, l_run));
  };

  // ---- tile fetch: every wave moves 2 KiB of each K and V tile ------------
  // DMA instruction i (0..1) of wave w fills LDS bytes [(2w + i) KiB, +1 KiB)
  // of the slot: key rows 8w + 4i .. +3 (K, dense V) or dimension rows
  // 16w + 8i .. +7 (paged V^T).  Each lane picks the global chunk whose
  // swizzled position is its own LDS position.
  const int rs = PAGED ? HD * 2 : p.Hkv * HD * 2;   // bytes between key rows
  int koff[2], voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * wave + 4 * i + (lane >> 4), pos = lane & 15;
    koff[i] = r * rs + 16 * k_pos(r, pos);
    if constexpr (PAGED) {
      const int d = 16 * wave + 8 * i + (lane >> 3), pv = lane & 7;
      voff[i] = d * (BN * 2) + 16 * vp_pos(d, pv);
    } else {
      voff[i] = r * rs + 16 * vd_pos(r, pos);
    }
  }
  const int32_t *table =
      PAGED ? p.block_table + ((size_t)b * p.Hkv + g) * p.max_blocks : nullptr;
  auto block_of = [&](int tile) __attribute__((always_inline)) -> int {
    if constexpr (PAGED) return tile < p.max_blocks ? ((const const_i32 *)table)[tile] : -1;
    return 0;
  };
  auto tile_rsrc = [&](const void *base, int tile, int blk, bool check) __attribute__((always_inline)) -> u32x4 {
    const bf16 *src = static_cast<const bf16 *>(base);
    if constexpr (PAGED) {
      const bool ok = blk >= 0 && blk < p.n_blocks;
      if (check && wave == 0 && lane == 0 && p.dev_status) {
        if (!ok)
          p.dev_status[0] = 2;
        else if (((const const_i32 *)p.block_head)[blk] != p.kv_head_base + g)
          p.dev_status[0] = 1;
      }
      return rsrc_words(src + (size_t)(ok ? blk : 0) * (TILE / 2), ok ? TILE : 0);
    } else {
      // the range ends at key row Sk of this batch: later rows read as zero
      const size_t first = (((size_t)b * p.Sk + (size_t)tile * BN) * p.Hkv + g) * HD;
      const long long bytes = ((long long)(p.Sk - tile * BN) * p.Hkv - g) * HD * 2;
      return rsrc_words(src + first, bytes > 0x7FFFFFFFLL ? 0x7FFFFFFF : (int)bytes);
    }
  };
  auto issue_k = [&](int t, int blk) __attribute__((always_inline)) {
    const u32x4 r = tile_rsrc(p.k, t, blk, true);
    char *dst = smem + kslot(t) + wave * 2048;
    dma_to_lds_16(r, dst, koff[0]);
    dma_to_lds_16(r, dst + 1024, koff[1]);
  };
  auto issue_v = [&](int t, int blk) __attribute__((always_inline)) {
    const u32x4 r = tile_rsrc(p.v, t, blk, false);
    char *dst = smem + vslot(t) + wave * 2048;
    dma_to_lds_16(r, dst, voff[0]);
    dma_to_lds_16(r, dst + 1024, voff[1]);
  };

  // ---- prologue: K_0..K_3, V_0, V_1 in flight, S_0 -------------------------
  for (int t = 0; t < KA && t < n_tiles; ++t) issue_k(t, block_of(t));
  for (int t = 0; t < VA && t < n_tiles; ++t) issue_v(t, block_of(t));
  int blk_k = block_of(KA), blk_v = block_of(VA);
  wait_vmcnt<0>();
  barrier_no_wait();
  if (wave_tiles > 0) s_plain(0, S[0], false);
  if (1 < wave_tiles) {
#pragma unroll
    for (int i = 0; i < NPK; ++i) kpre[i] = read_k(kslot(1), i);
  }
  // every wave is done with K_0 before iteration 0 refills its slot with K_KA
  barrier_no_wait();

  // Per-iteration tile fetch and the wait that publishes the previous
  // iteration's tiles at this iteration's barrier.
  auto fetch = [&](int j) __attribute__((always_inline)) -> int {
    const bool fk = j + KA < n_tiles, fv = j + VA < n_tiles;
    if (fk) issue_k(j + KA, blk_k);
    if (fv) issue_v(j + VA, blk_v);
    if (fk) blk_k = block_of(j + KA + 1);
    if (fv) blk_v = block_of(j + VA + 1);
    return 2 * (int)fk + 2 * (int)fv;   // DMA instructions issued by this wave
  };
  auto finish = [&](int j, int issued) __attribute__((always_inline)) {
    // DMAs of iteration j-1 have landed (this iteration's may still fly)
    if (issued == 4)
      wait_vmcnt<4>();
    else if (issued == 2)
      wait_vmcnt<2>();
    else
      wait_vmcnt<0>();
    if (PAGED) asm volatile("" ::"s"(blk_k), "s"(blk_v));   // block ids land here
    // first operands of the next iteration, read while waiting at the barrier
    if (j < wave_tiles) {
#pragma unroll
      for (int i = 0; i < NPV; ++i) vpre[i] = read_v(vslot(j), i);
    }
    if (j + 2 < wave_tiles) {
#pragma unroll
      for (int i = 0; i < NPK; ++i) kpre[i] = read_k(kslot(j + 2), i);
    }
    barrier_no_wait();
  };

  // Interleaved iteration j (needs j >= 1, j + 1 < wave_tiles, no mask):
  // P_{j-1} V_{j-1}, softmax(S_j) and S_{j+1} in one instruction stream.
  auto fused = [&](int j, auto par_tag) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_tag)::value;
    f32x16 (&sc)[2] = S[PAR];
    f32x16 (&sn)[2] = S[PAR ^ 1];
    bf16x8 (&pc)[4] = P[PAR];
    const bf16x8 (&pp)[4] = P[PAR ^ 1];
    const int issued = fetch(j);
    const int vs = vslot(j - 1), ks = kslot(j + 1);
    // The iteration is written as 32 MFMA slots, each fenced off from the
    // next: slot i issues MFMA i (16 of P V, then 16 of K Q^T), the LDS read
    // of the operand used four slots later, and a fixed share of the
    // softmax VALU work (the row max in slots 0-4, then the 16 bf16 pairs of
    // P with their exp2, pack and row-sum steps spread over slots 5-30).
    bf16x8 op[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      op[i] = vpre[i];
      op[16 + i] = kpre[i];
    }
    float t[11], mxv = 0.f, alpha = 1.f, psum = 0.f;
    bool grow = false;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int nx = i + 4;   // operand read in this slot
      if (nx < 16)
        op[nx] = read_v(vs, nx);
      else if (nx >= 20 && nx < 32)
        op[nx] = read_k(ks, nx - 16);
      if (i == 16) sn[0] = sn[1] = f32x16{};
      if (i < 16)
        acc[i & 3] = mfma_32x32x16(op[i], pp[i >> 2], acc[i & 3]);
      else
        sn[i & 1] = mfma_32x32x16(op[i], qf[(i - 16) >> 1], sn[i & 1]);
      // -- VALU share of slot i --
      if (i < 3) {   // 11 partial maxima of three (two for the last) scores
#pragma unroll
        for (int q = 4 * i; q < 4 * i + 4 && q < 11; ++q) {
          const int a = 3 * q, b2 = 3 * q + 1, c = 3 * q + 2;
          t[q] = q < 10 ? fmaxf(fmaxf(sc[a >> 4][a & 15], sc[b2 >> 4][b2 & 15]), sc[c >> 4][c & 15])
                        : fmaxf(sc[1][14], sc[1][15]);
        }
      } else if (i == 3) {
        mxv = fmaxf(fmaxf(fmaxf(fmaxf(t[0], t[1]), t[2]), fmaxf(fmaxf(t[3], t[4]), t[5])),
                    fmaxf(fmaxf(fmaxf(t[6], t[7]), t[8]), fmaxf(t[9], t[10])));
      } else if (i == 4) {
        const float mx2 = pair_max32(mxv) * c2;
        grow = mx2 > m2 + kRescaleLog2;
        const float m_new = grow ? mx2 : m2;
        alpha = fast_exp2(m2 - m_new);   // 1 where the max did not move
        m2 = m_new;
        psum = l_run * alpha;
      } else {
#pragma unroll
        for (int pr = 0; pr < 16; ++pr) {
          if (i != 5 + (pr * 27) / 16) continue;
          // pair pr = scores 2pr, 2pr+1 -> word (pr & 3) of P operand pr >> 2
          const int hf = pr >> 3, r = 2 * (pr & 7), u = pr >> 2;
          const float p0 = fast_exp2(fmaf(sc[hf][r], c2, -m2));
          const float p1 = fast_exp2(fmaf(sc[hf][r + 1], c2, -m2));
          pc[u][2 * (pr & 3)] = to_bf16(p0);
          pc[u][2 * (pr & 3) + 1] = to_bf16(p1);
          psum = add_bf16_pair(as_u32x4(pc[u])[pr & 3], psum);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run = psum;
    // P_j and l are produced in this iteration, not sunk into the next one
#pragma unroll
    for (int u = 0; u < 4; ++u) asm volatile("" ::"v"(pc[u]));
    asm volatile("" ::"v"(l_run));
    if (__ballot(grow)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;   // after P_{j-1} V_{j-1}
    }
    finish(j, issued);
  };

  // Plain iteration j: whatever of P_{j-1} V_{j-1}, softmax(S_j), S_{j+1}
  // this wave still has, one after the other.
  auto plain = [&](int j, auto par_tag) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_tag)::value;
    const int issued = fetch(j);
    if (j >= 1 && j - 1 < wave_tiles) pv_plain(j - 1, P[PAR ^ 1]);
    if (j < wave_tiles) softmax_plain(j, S[PAR], P[PAR]);
    if (j + 1 < wave_tiles) s_plain(j + 1, S[PAR ^ 1], true);
    finish(j, issued);
  };

  // Iterations 1 .. fused_end-1 need no mask and have all three parts.
  int fused_end = min(n_keys / BN, wave_tiles - 1);
  if (CAUSAL) fused_end = min(fused_end, (qoff + row0 + 1) / BN);
  plain(0, Int<0>{});
  int j = 1;
#pragma clang loop unroll(disable)
  for (; j + 1 < fused_end; j += 2) {
    fused(j, Int<1>{});
    fused(j + 1, Int<0>{});
  }
#pragma clang loop unroll(disable)
  for (; j <= n_tiles; j += 2) {
    plain(j, Int<1>{});
    if (j + 1 <= n_tiles) plain(j + 1, Int<0>{});
  }

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

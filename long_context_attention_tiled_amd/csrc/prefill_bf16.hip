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
constexpr int WD = 1;                   // DMAs are waited for WD iterations after issue
constexpr int KA = WD + 3;              // iteration j fetches K_{j+KA}
constexpr int VA = WD + 1;              // iteration j fetches V_{j+VA}
constexpr int NKS = KA;                 // K ring slots
constexpr int NVS = VA + 2;             // V ring slots (after the K slots)
constexpr int VBASE = NKS * TILE;       // LDS byte offset of the V ring
constexpr int LA = 2;                   // operands are read LA MFMA slots before their use
constexpr int NPV = LA;                 // P V operands read before the barrier
constexpr int NPK = LA;                 // K Q^T operands read before the barrier
// Every iteration issues the same DMA count per DMA wave; iteration j ends by
// waiting for those issued in iteration j-WD and earlier, and the barrier
// then publishes them.  K_t is read from the end of iteration t-2
// (first operands) to iteration t-1, V_t from the end of iteration t to
// iteration t+1; a slot is refilled (K_{t+NKS} in iteration t+NKS-KA,
// V_{t+NVS} in iteration t+NVS-VA) only after its last reader's barrier.
static_assert(KA >= WD + 3 && VA >= WD + 1, "tiles are published before their first read");
static_assert(NKS >= KA && NVS >= VA + 2, "a slot is refilled only after its last reader");
static_assert((NKS + NVS) * 16384 <= 160 * 1024, "LDS");
// Waves that issue the tile DMAs: the four older ones, 4 KiB of each tile
// apiece (see the fetch below).
constexpr int NDW = 4;

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
// The interleaved iterations skip the tile maximum altogether: they
// exponentiate against the running m as it stands and check the tile's row
// sum afterwards.  Every exponential is at most the row sum, so a sum at or
// below this bound (2^16) proves all of them are; fp32 and bf16 hold such
// values with full relative precision, and O and l stay within fp32 range
// for any realistic key count.  A larger sum (or inf) makes the wave redo
// the tile with the exact maximum before P is used.
constexpr float kSumLimit = 65536.0f;

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
// Tile movement: iteration j fetches K_{j+KA} and V_{j+VA} (the DMA waves
// share each tile) and ends by waiting for the DMAs it issued WD
// iterations earlier, so a tile has WD iterations to arrive.  A ring slot is
// refilled one iteration after its last reader.  Before the barrier a wave
// already reads the first operands of the next iteration (V_j for P_j V_j
// and K_{j+2} for S_{j+2}).
// Tiles that need the causal/length mask, and the first and last
// iterations, take a plain sequential path instead of the interleaved one.
// LIMITS (dense, with CAUSAL): row i of batch b sees keys [0, key_limit[b][i])
// instead of [0, i]; the limits must not decrease along the rows.
template <bool PAGED, bool CAUSAL, bool LIMITS = false>
__global__ __launch_bounds__(NT) void prefill_kernel(PrefillParams p, int heads_per_wg,
                                                     int head_slices, int n_qblk) {
  static_assert(!LIMITS || (CAUSAL && !PAGED), "key limits replace the dense causal rule");
  __shared__ __attribute__((aligned(1024))) char smem[(NKS + NVS) * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31;   // query column of this lane within the wave's 32 rows
  const int gq = lane >> 5;   // which 8-wide half of each 16-long K slice

  // ---- workgroup -> (query block, batch, KV head, head slice) -------------
  const int per_q = p.B * p.Hkv * head_slices;
  const int item = CAUSAL && !PAGED ? xcd_item(blockIdx.x, per_q, n_qblk) : (int)blockIdx.x;
  int qblk = item / per_q;
  if (CAUSAL) qblk = n_qblk - 1 - qblk;   // longest rows first
  int rem = item % per_q;
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
  int first_keys = n_keys;   // keys visible to every row of this wave (LIMITS)
  if constexpr (LIMITS) {
    // keys visible to query row r, clamped to the key count
    auto row_keys = [&](int r) -> int {
      return min(max(p.key_limit[(size_t)b * p.Sq + r], 0), n_keys);
    };
    wave_keys = row_keys(min(row0 + 31, p.Sq - 1));
    wg_keys = row_keys(min(qblk * rows_wg + rows_wg - 1, p.Sq - 1));
    first_keys = row_keys(min(row0, p.Sq - 1));
  } else if (CAUSAL) {
    wave_keys = min(n_keys, qoff + min(row0 + 31, p.Sq - 1) + 1);
    wg_keys = min(n_keys, qoff + min(qblk * rows_wg + rows_wg - 1, p.Sq - 1) + 1);
  }
  if (row0 >= p.Sq) wave_keys = 0;
  const int n_tiles = (wg_keys + BN - 1) / BN;
  const int wave_tiles = (wave_keys + BN - 1) / BN;

  // No row of this workgroup sees a key of this shard (limits do not
  // decrease, so the last row decides; the test is workgroup-uniform):
  // merging an empty partial into the running result changes nothing.
  if (LIMITS && p.accumulate && wg_keys == 0) return;

  // ---- this wave's 32 query rows -> registers (B operand of S^T = K Q^T) --
  // qf[s] = dims 16s + 8gq .. +7 of query row row0 + lr, multiplied by
  // scale * log2(e) and rounded to bf16, so that the MFMAs produce scores
  // already in log2 units (the softmax uses exp2).  Rows past the end
  // repeat the last row (finite data) and are never stored.
  const float c2 = p.scale * kLog2e;
  const int qrow = row0 + lr;
  bf16x8 qf[8];
  {
    const int qr = min(qrow, p.Sq - 1);
    const bf16 *qp = static_cast<const bf16 *>(p.q) + (((size_t)b * p.Sq + qr) * p.Hq + h) * HD;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(ld_global_16(qp + 16 * s + 8 * gq));
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][e] = to_bf16((float)qf[s][e] * c2);
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
  // The V ring starts at byte VBASE; keeping VBASE in the per-lane base
  // registers leaves slot + operand offsets below 64 KiB, so every V read
  // below is base register + immediate offset.
#pragma unroll
  for (int i = 0; i < 4; ++i) va[i] = opaque(va[i] + VBASE);
  // operand i = 4u + db of P V for the V tile in LDS slot `vs` (byte offset
  // of the slot from the start of LDS)
  auto read_v = [&](int vs, int i) __attribute__((always_inline)) -> bf16x8 {
    const int u = i >> 2, db = i & 3;
    if constexpr (PAGED) {
      return *reinterpret_cast<const bf16x8 *>(smem + (vs - VBASE) + va[u ^ (2 * (db & 1))] + 4096 * db);
    } else {
      const char *a = smem + (vs - VBASE) + va[db] + 4096 * u;
      const u32x2 lo = lds_read_tr16(a), hi = lds_read_tr16(a + 1024);
      return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
    }
  };
  // operand i = 2s + hf of S = K Q^T for the K tile in LDS slot `ks`
  auto read_k = [&](int ks, int i) __attribute__((always_inline)) -> bf16x8 {
    return *reinterpret_cast<const bf16x8 *>(smem + ks + kaddr[i >> 1] + 8192 * (i & 1));
  };
  // Ring slot byte offsets advance by one slot per iteration (no division).
  auto next_k = [](int x) { return x + TILE == NKS * TILE ? 0 : x + TILE; };
  auto next_v = [](int x) { return x + TILE == (NKS + NVS) * TILE ? NKS * TILE : x + TILE; };

  // last key this lane's row may see
  int qlast;
  if constexpr (LIMITS)
    qlast = min(max(p.key_limit[(size_t)b * p.Sq + min(qrow, p.Sq - 1)], 0), n_keys) - 1;
  else
    qlast = CAUSAL ? min(n_keys - 1, qoff + qrow) : n_keys - 1;

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
  // Score tiles hold (scale * log2 e) * s - m2 (or - 0 while m2 is -inf):
  // every S^T accumulator chain starts from negm, a register tile filled
  // with that shift, so the softmax exponentiates MFMA outputs directly.
  // When m2 rises, a score tile already computed for a later key tile is
  // moved by the same amount.
  f32x16 negm = f32x16{};
  auto set_shift = [&]() __attribute__((always_inline)) {
    const float sh = m2 == -INFINITY ? 0.f : -m2;
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = sh;
  };

  // ---- plain (sequential) pieces, used for edge iterations ----------------
  auto pv_plain = [&](int t, int vs, const bf16x8 (&pp)[4]) __attribute__((always_inline)) {
    const int nv = n_keys - t * BN;   // valid keys in this tile
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      bf16x8 a = i < NPV ? vpre[i < NPV ? i : 0] : read_v(vs, i);
      if (PAGED && nv < BN) a = mask_keys(a, 16 * (i >> 2) + 8 * gq, nv);
      acc[i & 3] = mfma_32x32x16(a, pp[i >> 2], acc[i & 3]);
    }
  };
  auto s_plain = [&](int ks, f32x16 (&sn)[2], bool use_pre) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bf16x8 a = (i < NPK && use_pre) ? kpre[i < NPK ? i : 0] : read_k(ks, i);
      sn[i & 1] = mfma_32x32x16(a, qf[i >> 1], i < 2 ? negm : sn[i & 1]);
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
  // exp2(score - d) of half hf of a score tile into P (bf16), returning the
  // partial row sum
  auto exp_half = [&](const f32x16 (&sc)[2], bf16x8 (&pc)[4], int hf, float d,
                      float psum) __attribute__((always_inline)) -> float {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pc[2 * hf + u][e] = to_bf16(fast_exp2(sc[hf][8 * u + e] - d));
      const u32x4 w = as_u32x4(pc[2 * hf + u]);
#pragma unroll
      for (int e = 0; e < 4; ++e) psum = add_bf16_pair(w[e], psum);
    }
    return psum;
  };
  auto softmax_plain = [&](int t, f32x16 (&sc)[2], bf16x8 (&pc)[4]) __attribute__((always_inline)) {
    const int key0 = t * BN;
    const bool need_mask = LIMITS ? key0 + BN > first_keys
                                  : (key0 + BN > n_keys) || (CAUSAL && key0 + BN - 1 > qoff + row0);
    if (need_mask) {
      const int lim = qlast;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = key0 + 16 * (r >> 3) + 8 * gq + (r & 7);
        if (kk > lim) sc[0][r] = -INFINITY;
        if (kk + 32 > lim) sc[1][r] = -INFINITY;
      }
    }
    const float sh = m2 == -INFINITY ? 0.f : m2;   // shift the tile was computed with
    const float mx2 = tile_max(sc) + sh;
    const bool grow = mx2 > m2 + kRescaleLog2;
    if (__ballot(grow)) {
      const float m_new = grow ? mx2 : m2;
      const float alpha = grow ? fast_exp2(m2 - m_new) : 1.f;
      m2 = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;
      set_shift();
    }
    const float d = (m2 == -INFINITY) ? 0.f : m2 - sh;
    l_run = exp_half(sc, pc, 1, d, exp_half(sc, pc, 0, d, l_run));
  };

  // ---- tile fetch: NDW waves move 16/NDW KiB of each K and V tile ---------
  // With NDW = 4 only the older wave of each SIMD (waves w and w+4 share one)
  // issues DMAs: it wins issue arbitration and finishes its MFMA slots
  // first, so it fetches while the younger one starts computing.  Each lane
  // picks the global chunk whose swizzled position is its own LDS position.
  //  * K and dense V: DMA instruction i of wave w fills key rows
  //    16 i + 4 w .. +3, LDS bytes [4096 i + 1024 w, +1 KiB) of the slot.
  //    Rows 16 apart share one chunk permutation, so a wave's instructions
  //    differ only by the uniform source stride of 16 rows, added to one
  //    base offset register per tensor.
  //  * Paged V^T: instruction i of wave w fills dimension rows
  //    32 i + 8 w .. +7, LDS bytes [4096 i + 1024 w, +1 KiB).  Rows 64 apart
  //    share one chunk permutation, so instructions i and i + 2 differ by a
  //    uniform 8 KiB of source: two offset registers per wave.
  constexpr int DPW = TILE / 1024 / NDW;   // 1 KiB pieces per DMA wave, tile and tensor
  static_assert(DPW * NDW * 4 == BN && NDW * 4 == 16, "row mapping of the K / dense V DMAs");
  const bool dma_wave = wave < NDW;
  const int rs = PAGED ? HD * 2 : p.Hkv * HD * 2;   // bytes between key rows
  const int rstep = 16 * rs;                         // source bytes between a wave's DMAs
  static_assert(!PAGED || DPW == 4, "row mapping of the paged V^T DMAs");
  int kbase, vbase = 0, vodd = 0;
  {
    const int r = 4 * wave + (lane >> 4), pos = lane & 15;
    kbase = r * rs + 16 * k_pos(r, pos);
    if constexpr (PAGED) {
      const int d = 8 * wave + (lane >> 3), pv = lane & 7;
      vbase = d * (BN * 2) + 16 * vp_pos(d, pv);
      vodd = (d + 32) * (BN * 2) + 16 * vp_pos(d + 32, pv);
    } else {
      vbase = r * rs + 16 * vd_pos(r, pos);
    }
  }
  const int32_t *table =
      PAGED ? p.block_table + ((size_t)b * p.Hkv + g) * p.max_blocks : nullptr;
  auto block_of = [&](int tile) __attribute__((always_inline)) -> int {
    if constexpr (PAGED) return tile < p.max_blocks ? ((const const_i32 *)table)[tile] : -1;
    return 0;
  };
  // Tile sources.  Dense: a running descriptor per tensor whose range ends at
  // key row Sk of this batch (later rows read as zero).  Paged: one block.
  // Tiles at or past n_tiles get an empty range: their DMA reads nothing and
  // writes zeros into a slot that is free anyway, so every iteration issues
  // the same number of DMA instructions.
  struct Stream {
    const char *base;   // first byte of the next tile to fetch
    int rows_left;      // key rows of this batch from there on (Sk - 64 tile)
  };
  const long long tstride = (long long)BN * p.Hkv * HD * 2;   // bytes per dense tile
  auto dense_stream = [&](const void *t0) __attribute__((always_inline)) -> Stream {
    const size_t first = (((size_t)b * p.Sk) * p.Hkv + g) * HD;
    return Stream{static_cast<const char *>(t0) + first * 2, p.Sk};
  };
  Stream ks_stream = dense_stream(p.k), vs_stream = dense_stream(p.v);
  auto issue = [&](Stream &st, int tile, int blk, int slot_off,
                   bool is_k) __attribute__((always_inline)) {
    u32x4 r;
    if constexpr (PAGED) {
      const bf16 *src = static_cast<const bf16 *>(is_k ? p.k : p.v);
      const bool ok = blk >= 0 && blk < p.n_blocks;   // reported by the scan above
      r = rsrc_words(src + (size_t)(ok ? blk : 0) * (TILE / 2), ok && tile < n_tiles ? TILE : 0);
    } else {
      // the range ends at key row Sk of this batch (later rows read as zero)
      // or after the tile, whichever comes first
      const int nb = tile < n_tiles ? (min(st.rows_left, BN) * p.Hkv - g) * (HD * 2) : 0;
      r = rsrc_words(st.base, nb);
      st.base += tstride;
      st.rows_left -= BN;
    }
    if (PAGED && !is_k) {
      const int b0 = opaque(vbase), b1 = opaque(vodd);
      char *dst = smem + slot_off + wave * 1024;
#pragma unroll
      for (int i = 0; i < DPW; ++i)
        dma_to_lds_16(r, dst + 4096 * i, (i & 1 ? b1 : b0) + (i >> 1) * (64 * BN * 2));
    } else {
      // the per-instruction offsets are recomputed here (one add each)
      // rather than held in registers across the loop
      const int base = opaque(is_k ? kbase : vbase);
      char *dst = smem + slot_off + wave * 1024;
#pragma unroll
      for (int i = 0; i < DPW; ++i) dma_to_lds_16(r, dst + 4096 * i, base + i * rstep);
    }
  };

  // Paged: wave 0 checks the ids and tags of all n_tiles blocks once, 64 at
  // a time; an id out of range is replaced by an empty range (zeros) when
  // its tile is fetched.
  if (PAGED && wave == 0 && p.dev_status) {
    bool bad_id = false, bad_tag = false;
    for (int t = lane; t < n_tiles; t += 64) {
      const int blk = table[t];
      const bool ok = blk >= 0 && blk < p.n_blocks;
      bad_id |= !ok;
      bad_tag |= ok && p.block_head[blk] != p.kv_head_base + g;
    }
    const bool any_id = __ballot(bad_id) != 0, any_tag = __ballot(bad_tag) != 0;
    if (lane == 0 && (any_id || any_tag)) p.dev_status[0] = any_id ? 2 : 1;
  }

  // ---- prologue: K_0..K_{KA-1}, V_0..V_{VA-1} in flight, then S_0 --------
  if (dma_wave) {
#pragma unroll
    for (int t = 0; t < KA; ++t) issue(ks_stream, t, block_of(t), t * TILE, true);
#pragma unroll
    for (int t = 0; t < VA; ++t) issue(vs_stream, t, block_of(t), (NKS + t) * TILE, false);
  }
  int blk_k = block_of(KA), blk_v = block_of(VA);
  // S_0 and the operand reads before the next barrier need K_0 and K_1
  // only, so the first barrier publishes just those; the other prologue
  // tiles keep flying while S_0 is computed.  Waves that issued no DMA have
  // nothing in flight.
  static_assert(KA >= 2, "K_0 and K_1 are waited for separately");
  wait_vmcnt<(KA - 2 + VA) * DPW>();
  barrier_no_wait();
  if (wave_tiles > 0) s_plain(0, S[0], false);   // K_0 in slot 0
  if (1 < wave_tiles) {
#pragma unroll
    for (int i = 0; i < NPK; ++i) kpre[i] = read_k(TILE, i);
  }
  // Iteration 0 reads operands of V_0 and K_2 before its own barrier, and
  // every wave's DMAs wrote rows of them: all prologue DMAs have landed
  // before this barrier, which publishes them.  It also keeps iteration 0
  // from refilling K_0's slot while a wave still reads K_0.
  wait_vmcnt<0>();
  barrier_no_wait();

  // kc: K slot of tile j (= slot of K_{j+KA}, refilled in iteration j);
  // vc: V slot of tile j-2 (= slot of V_{j+VA}, refilled in iteration j).
  // The interleaved loop below uses the same positions as constants.
  int kc = 0, vc = (NKS + NVS - 2) * TILE;
  static_assert(NKS == KA && NVS == VA + 2, "slot bookkeeping below");
  static_assert(NKS == 4 && NVS == 4, "the interleaved loop is unrolled over a 4-slot ring");

  // Per-iteration tile fetch (2 DPW DMA instructions per DMA wave, always) into the
  // given K and V slots, and the wait that publishes the tiles fetched WD
  // iterations earlier, followed by the first operand reads of the next
  // iteration (V_j and K_{j+2}, from the given slots).
  auto fetch = [&](int j, int kdst, int vdst) __attribute__((always_inline)) {
    if (dma_wave) {
      issue(ks_stream, j + KA, blk_k, kdst, true);
      issue(vs_stream, j + VA, blk_v, vdst, false);
      blk_k = block_of(j + KA + 1);
      blk_v = block_of(j + VA + 1);
    }
  };
  auto finish = [&](int j, int v_next, int k_next2) __attribute__((always_inline)) {
    wait_vmcnt<2 * DPW * WD>();   // DMAs of iterations j-WD+1 .. j may still fly
    if (PAGED) asm volatile("" ::"s"(blk_k), "s"(blk_v));   // block ids land here
    if (j < wave_tiles) {
#pragma unroll
      for (int i = 0; i < NPV; ++i) vpre[i] = read_v(v_next, i);
    }
    if (j + 2 < wave_tiles) {
#pragma unroll
      for (int i = 0; i < NPK; ++i) kpre[i] = read_k(k_next2, i);
    }
    barrier_no_wait();
  };

  // Interleaved iteration j (needs j >= 1, j + 1 < wave_tiles, no mask):
  // P_{j-1} V_{j-1}, softmax(S_j) and S_{j+1} in one instruction stream.
  // R = j % 4 is the ring position, so every LDS offset is a constant.
  auto fused = [&](int j, auto par_tag, auto ring_tag) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_tag)::value;
    constexpr int R = decltype(ring_tag)::value;
    f32x16 (&sc)[2] = S[PAR];
    f32x16 (&sn)[2] = S[PAR ^ 1];
    bf16x8 (&pc)[4] = P[PAR];
    const bf16x8 (&pp)[4] = P[PAR ^ 1];
    constexpr int kdma = R * TILE, ks = ((R + 1) % NKS) * TILE, kpre_s = ((R + 2) % NKS) * TILE;
    constexpr int vdma = (NKS + (R + VA) % NVS) * TILE, vs = (NKS + (R + NVS - 1) % NVS) * TILE,
                  vpre_s = (NKS + R) * TILE;
    fetch(j, kdma, vdma);
    // The iteration is written as 32 MFMA slots, each fenced off from the
    // next: slot i issues MFMA i (16 of P V, then 16 of K Q^T), the LDS read
    // of the operand used LA slots later, and a fixed share of the softmax
    // VALU work: pair pr of P (scores 2pr, 2pr+1 -> word pr & 3 of operand
    // pr >> 2) has its first score exponentiated in slot 2pr and its second
    // in slot 2pr+1; it is packed to bf16 in slot 2pr+2 and added to the row
    // sum in slot 2pr+3, so every slot carries one exp2 and one more VALU
    // instruction, and no step waits for the one before it inside a slot.
    // The scores arrive scaled and shifted by the running maximum (negm);
    // no tile maximum is taken here (see kSumLimit).
    bf16x8 op[32];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      op[i] = vpre[i];
      op[16 + i] = kpre[i];
    }
    float ts = 0.f;     // this tile's row sum (this lane's keys)
    float xs[2][2];     // pairs in flight between the exp2 and pack steps
    auto pack_pair = [&](auto pr_tag) __attribute__((always_inline)) {
      constexpr int pr = decltype(pr_tag)::value;
      constexpr int u = pr >> 2;
      pc[u][2 * (pr & 3)] = to_bf16(xs[pr & 1][0]);
      pc[u][2 * (pr & 3) + 1] = to_bf16(xs[pr & 1][1]);
    };
    auto sum_pair = [&](auto pr_tag) __attribute__((always_inline)) {
      constexpr int pr = decltype(pr_tag)::value;
      ts = add_bf16_pair(as_u32x4(pc[pr >> 2])[pr & 3], ts);
    };
    static_for<32>([&](auto slot_tag) __attribute__((always_inline)) {
      constexpr int i = decltype(slot_tag)::value;
      constexpr int nx = i + LA;   // operand read in this slot
      if constexpr (nx < 16)
        op[nx] = read_v(vs, nx);
      else if constexpr (nx >= 16 + NPK && nx < 32)
        op[nx] = read_k(ks, nx - 16);
      if constexpr (i < 16)
        acc[i & 3] = mfma_32x32x16(op[i], pp[i >> 2], acc[i & 3]);
      else if constexpr (i < 18)
        sn[i & 1] = mfma_32x32x16(op[i], qf[(i - 16) >> 1], negm);
      else
        sn[i & 1] = mfma_32x32x16(op[i], qf[(i - 16) >> 1], sn[i & 1]);
      // -- VALU share of slot i --
      constexpr int pr = i >> 1;
      constexpr int hf = pr >> 3, r = 2 * (pr & 7) + (i & 1);
      xs[pr & 1][i & 1] = fast_exp2(sc[hf][r]);
      if constexpr (pr >= 1) {
        if constexpr ((i & 1) == 0)
          pack_pair(Int<pr - 1>{});
        else
          sum_pair(Int<pr - 1>{});
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    pack_pair(Int<15>{});
    sum_pair(Int<15>{});
    // P_j and l are produced in this iteration, not sunk into the next one
#pragma unroll
    for (int u = 0; u < 4; ++u) asm volatile("" ::"v"(pc[u]));
    const float l_prev = l_run;
    l_run = l_prev + ts;
    asm volatile("" ::"v"(l_run));
    if (__ballot(!(ts <= kSumLimit))) {
      // rare: some exponential may exceed the bound; redo the tile against
      // its exact maximum and rescale O (which now holds P_{j-1} V_{j-1}).
      // m2 is finite here (every row of the wave has seen key tile 0), and
      // the tile's scores are relative to it.
      const float dm = fmaxf(tile_max(sc), 0.f);
      const float alpha = fast_exp2(-dm);
      m2 += dm;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;
      l_run = exp_half(sc, pc, 1, dm, exp_half(sc, pc, 0, dm, l_prev * alpha));
      // the next tile's scores were computed against the old maximum
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sn[0][r] -= dm;
        sn[1][r] -= dm;
      }
      set_shift();
    }
    finish(j, vpre_s, kpre_s);
  };

  // Plain iteration j: whatever of P_{j-1} V_{j-1}, softmax(S_j), S_{j+1}
  // this wave still has, one after the other (ring positions at run time).
  auto plain = [&](int j, auto par_tag) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_tag)::value;
    const int vs = next_v(vc), ks = next_k(kc);   // V_{j-1}, K_{j+1}
    fetch(j, kc, vc);
    if (j >= 1 && j - 1 < wave_tiles) pv_plain(j - 1, vs, P[PAR ^ 1]);
    if (j < wave_tiles) softmax_plain(j, S[PAR], P[PAR]);
    if (j + 1 < wave_tiles) s_plain(ks, S[PAR ^ 1], true);
    finish(j, next_v(vs), next_k(ks));
    kc = next_k(kc);
    vc = next_v(vc);
  };

  // Iterations 1 .. fused_end-1 need no mask and have all three parts; the
  // interleaved loop takes them four at a time (ring positions 1, 2, 3, 0).
  int fused_end = min(n_keys / BN, wave_tiles - 1);
  if (LIMITS) fused_end = min(fused_end, first_keys / BN);
  else if (CAUSAL) fused_end = min(fused_end, (qoff + row0 + 1) / BN);
  plain(0, Int<0>{});
  int j = 1;
#pragma clang loop unroll(disable)
  for (; j + 3 < fused_end; j += 4) {
    fused(j, Int<1>{}, Int<1>{});
    fused(j + 1, Int<0>{}, Int<2>{});
    fused(j + 2, Int<1>{}, Int<3>{});
    fused(j + 3, Int<0>{}, Int<0>{});
  }
  // up to three more interleaved iterations (ring positions 1, 2, 3), so the
  // plain path runs only where it must (first tile, mask, last tiles)
  if (j < fused_end) {
    fused(j++, Int<1>{}, Int<1>{});
    if (j < fused_end) {
      fused(j++, Int<0>{}, Int<2>{});
      if (j < fused_end) fused(j++, Int<1>{}, Int<3>{});
    }
  }
  // back to run-time ring positions for the remaining iterations
  kc = (j % NKS) * TILE;
  vc = (NKS + (j + NVS - 2) % NVS) * TILE;
  if (!(j & 1) && j <= n_tiles) plain(j++, Int<0>{});
#pragma clang loop unroll(disable)
  for (; j <= n_tiles; j += 2) {
    plain(j, Int<1>{});
    if (j + 1 <= n_tiles) plain(j + 1, Int<0>{});
  }

  // ---- epilogue: divide by l once, store O (bf16) and LSE ----------------
  const float l_tot = pair_sum32(l_run);
  if (qrow < p.Sq) {
    float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16 *op = static_cast<bf16 *>(p.o) + (((size_t)b * p.Sq + qrow) * p.Hq + h) * HD;
    float *lp = p.lse + ((size_t)b * p.Hq + h) * p.Sq + qrow;
    float lse2 = l_tot > 0.f ? m2 + __log2f(l_tot) : -INFINITY;   // log2 units
    float w_prev = 0.f;
    if (LIMITS && p.accumulate) {
      // o / lse hold a normalised partial of this row over other keys: merge
      // with the log-sum-exp rescale (weights 2^(L - M), empty sides weigh 0)
      const float prev2 = *lp * kLog2e;
      const float M = fmaxf(prev2, lse2);
      if (M != -INFINITY) {
        w_prev = prev2 == -INFINITY ? 0.f : fast_exp2(prev2 - M);
        const float w_cur = lse2 == -INFINITY ? 0.f : fast_exp2(lse2 - M);
        const float den = w_prev + w_cur;
        inv = w_cur * inv / den;
        w_prev /= den;
        lse2 = M + __log2f(den);
      }
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int hp = 0; hp < 2; ++hp) {
        // acc[db] register 4 rq + e holds dim 32 db + 8 rq + 4 gq + e of this
        // lane's row.  One swap with lane l ^ 32 per value pair leaves
        // dims 32 db + 16 hp + 8 gq .. +7 in f[0..7], so each lane stores
        // 16 contiguous bytes (32 per row and instruction) instead of 8.
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const auto r = __builtin_amdgcn_permlane32_swap(
              __builtin_bit_cast(uint32_t, acc[db][4 * (2 * hp) + e] * inv),
              __builtin_bit_cast(uint32_t, acc[db][4 * (2 * hp + 1) + e] * inv), false, false);
          f[e] = __builtin_bit_cast(float, (uint32_t)r[0]);
          f[4 + e] = __builtin_bit_cast(float, (uint32_t)r[1]);
        }
        bf16x8 *dst = reinterpret_cast<bf16x8 *>(op + 32 * db + 16 * hp + 8 * gq);
        bf16x8 w;
        if (LIMITS && p.accumulate) {
          const bf16x8 prev = *dst;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            w[e] = to_bf16(f[e] + (w_prev > 0.f ? w_prev * (float)prev[e] : 0.f));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = to_bf16(f[e]);
        }
        *dst = w;
      }
    }
    if (p.lse && gq == 0) *lp = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
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
  } else if (p.key_limit) {
    hipLaunchKernelGGL((prefill_kernel<false, true, true>), grid, block, 0, stream, p,
                       heads_per_wg, head_slices, n_qblk);
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

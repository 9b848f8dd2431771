// Tiled exact attention with FP8 (OCP e4m3) scores on gfx950, head_dim 128.
//
// FA3's FP8 path ("Flash Attention and distributed inference", §18.5) runs
// the attention matmuls on 8-bit operands with block quantisation.  Here the
// score product S = Q K^T runs on the scaled FP8 matrix core instruction
// (v_mfma_scale_f32_32x32x64_f8f6f4), whose per-block power-of-two scales
// carry the block quantisation for free: each 32 head dims of a query row
// and of a key row have their own E8M0 scale (rule in fp8_block.h).  P V
// stays on bf16 MFMA with bf16 V and bf16 P.  Everything else is the bf16
// prefill: K/V tiles staged in LDS rings by DMA, S^T = K Q^T so that softmax
// statistics are lane-local, online softmax with a running max m and
// denominator l ("Flash Attention and distributed inference", §18.3),
// deferred division by l (§18.4), scores never leave registers.
//
// Inputs: q bf16 [B][S][Hq][128]; k8 e4m3 [B][S][Hkv][128] with k_scale E8M0
// [B][S][Hkv][4] (block i covers dims 32i .. 32i+31), as attn_quantize_fp8_blocks
// writes them; v bf16 [B][S][Hkv][128].  Each wave multiplies its query rows
// by scale * log2(e) in fp32 and quantises them per 32 dims with the same
// rule as it loads them, so the matrix core produces the softmax exponents
// (log2 units) directly.  With rotation signs (incoherent processing,
// hadamard.h) each query row is first rotated, and k8 holds the rotated K.
//
// The operand layout of the scaled FP8 MFMA is stated in prefill_fp8_common.h.
#include "device.h"
#include "fp8_block.h"
#include "kernels.h"
#include "prefill_fp8_common.h"

namespace lcat {
namespace {

constexpr int HD = 128;                 // head dimension
constexpr int BN = 64;                  // keys per tile
constexpr int NW = 8;                   // waves per workgroup
constexpr int NT = NW * 64;             // threads per workgroup
constexpr int KT = BN * HD;             // bytes of one e4m3 K tile [64][128]
constexpr int VT = BN * HD * 2;         // bytes of one bf16 V tile [64][128]
constexpr int ST = 1024;                // bytes of a K-scale slot (4 copies of 64 words)
constexpr int KA = 5;                   // iteration j fetches K_{j+KA}
constexpr int VA = 3;                   // iteration j fetches V_{j+VA}
constexpr int NKS = 6;                  // K (and K-scale) ring slots
constexpr int NVS = 6;                  // V ring slots
constexpr int VBASE = NKS * KT;         // LDS byte offset of the V ring
constexpr int SBASE = VBASE + NVS * VT; // LDS byte offset of the K-scale ring
constexpr int LDS_BYTES = SBASE + NKS * ST;
constexpr int LA = 2;                   // operands are read LA MFMA slots before their use
constexpr int NPV = LA;                 // P V operands read before the barrier
constexpr int NPK = 1;                  // K Q^T operands read before the barrier
constexpr int NDW = 4;                  // waves that issue the tile DMAs
constexpr int KDPW = KT / 1024 / NDW;   // code DMAs per DMA wave and K tile
constexpr int VDPW = VT / 1024 / NDW;   // DMAs per DMA wave and V tile
constexpr int DPI = KDPW + 1 + VDPW;    // DMAs per DMA wave and iteration
// Barriers come in pairs of iterations: only even iterations end with a DMA
// wait and a barrier.  A tile fetched in an odd iteration j is published at
// the end of j + 1, one fetched in an even iteration at the end of j + 2.
// K_i is first read at the end of iteration i - 2 (operands read ahead)
// and last read in iteration i - 1; V_i is first read at the end of
// iteration i and last read in iteration i + 1.  The fetch in iteration j
// follows the barrier of iteration j - 1 (j odd) or j - 2 (j even), and the
// slot it fills must have been read for the last time before that barrier.
static_assert(KA >= 5 && VA >= 3, "tiles are published before their first read");
static_assert(NKS >= KA + 1 && NVS >= VA + 3, "a slot is refilled after its last read");
static_assert(NKS == 6 && NVS == 6, "the interleaved loop is unrolled over a 6-slot ring");
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
static_assert(KDPW == 2 && VDPW == 4, "row mapping of the DMAs");

// e4m3 K tile: 64 key rows x 8 chunks of 16 dims (128 B rows).  Chunk c of
// row r sits at c ^ ((r >> 1) & 7): the 16 rows a quarter-wave reads for
// one operand chunk fall on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int k8_pos(int row, int c) { return c ^ ((row >> 1) & 7); }
// bf16 V rows: chunk c of row r at c ^ 4*(r & 3) (see the bf16 prefill).
__device__ __forceinline__ int vd_pos(int row, int c) { return c ^ ((row & 3) << 2); }

constexpr float kRescaleLog2 = 8.0f;    // lazy rescale threshold of the edge iterations
constexpr float kSumLimit = 65536.0f;   // row-sum bound of the interleaved iterations

// Schedule: as the bf16 prefill, iteration j interleaves
//   O^T += V_{j-1}^T P_{j-1}^T      (16 bf16 MFMA, operands from the V ring)
//   softmax of S_j -> P_j, m, l     (VALU)
//   S_{j+1}^T = K_{j+1} Q^T         (4 scaled FP8 MFMA, operands from the K ring)
// and fetches K_{j+KA} (codes and scales) and V_{j+VA}.  The four FP8 MFMAs
// each take as long as two bf16 ones and carry four of the softmax's 32
// exponentials; the sixteen bf16 ones carry one each.
template <bool CAUSAL>
__global__ __launch_bounds__(NT) void prefill_fp8_kernel(PrefillFp8Params p, int heads_per_wg,
                                                         int head_slices, int n_qblk) {
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31;   // query column of this lane within the wave's 32 rows
  const int gq = lane >> 5;   // which half of each operand block

  // ---- workgroup -> (query block, batch, KV head, head slice) -------------
  const int per_q = p.B * p.Hkv * head_slices;
  const int item = CAUSAL ? xcd_item(blockIdx.x, per_q, n_qblk) : (int)blockIdx.x;
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

  const int n_keys = p.S;
  int wave_keys = n_keys, wg_keys = n_keys;
  if (CAUSAL) {
    wave_keys = min(n_keys, min(row0 + 31, p.S - 1) + 1);
    wg_keys = min(n_keys, min(qblk * rows_wg + rows_wg - 1, p.S - 1) + 1);
  }
  if (row0 >= p.S) wave_keys = 0;
  const int n_tiles = (wg_keys + BN - 1) / BN;
  const int wave_tiles = (wave_keys + BN - 1) / BN;

  // ---- this wave's 32 query rows, scaled and quantised -> registers -------
  // qf[c] is the B operand of the MFMA over dims 64c .. 64c+63: bytes 0..15
  // hold dims 64c + 16 gq .. +15 and bytes 16..31 dims 64c + 32 + 16 gq .. +15
  // of query row row0 + lr, each multiplied by scale * log2(e) in fp32 and
  // divided by its block's power of two.  qsw holds the E8M0 scale of block
  // 2c + gq in byte 2c.  Rows past the end repeat the last row (finite data)
  // and are never stored.
  const float c2 = p.scale * kLog2e;
  const int qrow = row0 + lr;
  i32x8 qf[2];
  const bf16 *qrow_p =
      static_cast<const bf16 *>(p.q) + (((size_t)b * p.S + min(qrow, p.S - 1)) * p.Hq + h) * HD;
  const int qsw = p.rot.on ? quantize_query_row_rotated(qrow_p, gq, c2 * (1.0f / 128), p.rot, qf)
                           : quantize_query_row(qrow_p, gq, c2, qf);
#pragma unroll
  for (int c = 0; c < 2; ++c) asm volatile("" ::"v"(qf[c]));

  // ---- LDS operand addresses (within a slot) ------------------------------
  // K rows are read in a permuted order (bits 2 and 3 of the row swapped) so
  // that the score registers land in the B-operand order of P V; rows 32..63
  // sit 4 KiB further.  K operand (hf, c): chunks 4c + gq and 4c + 2 + gq of
  // row krow + 32 hf.
  const int krow = (lr & ~12) | ((lr & 4) << 1) | ((lr & 8) >> 1);
  int kaddr[2][2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) kaddr[c][pt] = krow * 128 + 16 * k8_pos(krow, 4 * c + 2 * pt + gq);
  // K-scale word of key row krow (+32 hf) in copy 0 of a scale slot
  const int saddr = opaque(SBASE + 4 * krow);
  // V^T operand (key step u, dim block db) via transposing reads, as in the
  // bf16 prefill; VBASE is folded into the base registers.
  int va[4];
  {
    const int q4 = (lane >> 2) & 3;
    const int r0 = 8 * (lane >> 5) + q4;
    const int c0 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) va[db] = opaque(VBASE + r0 * 256 + 16 * (4 * (db ^ q4) + c0) + 8 * (lane & 1));
  }
  auto read_v = [&](int vs, int i) __attribute__((always_inline)) -> bf16x8 {
    const int u = i >> 2, db = i & 3;
    const char *a = smem + (vs - VBASE) + va[db] + 4096 * u;
    const u32x2 lo = lds_read_tr16(a), hi = lds_read_tr16(a + 1024);
    return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
  };
  // K operand t = 2c + hf of S = K Q^T for the K tile in slot offset ks
  auto read_k = [&](int ks, int t) __attribute__((always_inline)) -> i32x8 {
    const int hf = t & 1, c = t >> 1;
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(smem + ks + kaddr[c][0] + 4096 * hf);
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(smem + ks + kaddr[c][1] + 4096 * hf);
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // Scale word of half hf for the K tile in K slot ks (natural block order),
  // shifted so that byte 2c holds block 2c + gq.
  auto read_ksw = [&](int ks, int hf) __attribute__((always_inline)) -> int {
    const int w = *reinterpret_cast<const int *>(smem + saddr + (ks / KT) * ST + 128 * hf);
    return (int)((uint32_t)w >> (8 * gq));
  };
  // ring slots of K_t and V_t
  auto k_slot = [](int t) { return (int)((unsigned)t % NKS) * KT; };
  auto v_slot = [](int t) { return VBASE + (int)((unsigned)t % NVS) * VT; };

  const int qlast = CAUSAL ? min(n_keys - 1, qrow) : n_keys - 1;

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  f32x16 S[2][2];
  bf16x8 P[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    S[a][0] = S[a][1] = f32x16{};
#pragma unroll
    for (int u = 0; u < 4; ++u) P[a][u] = bf16x8{};
  }
  bf16x8 vpre[NPV];
  i32x8 kpre[NPK];
  int kswpre[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < NPV; ++i) vpre[i] = bf16x8{};
#pragma unroll
  for (int i = 0; i < NPK; ++i) kpre[i] = i32x8{};
  float m2 = -INFINITY;
  float l_run = 0.f;
  f32x16 negm = f32x16{};
  auto set_shift = [&]() __attribute__((always_inline)) {
    const float sh = m2 == -INFINITY ? 0.f : -m2;
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = sh;
  };

  // ---- plain (sequential) pieces, used for edge iterations ----------------
  auto pv_plain = [&](int vs, const bf16x8 (&pp)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bf16x8 a = i < NPV ? vpre[i < NPV ? i : 0] : read_v(vs, i);
      acc[i & 3] = mfma_32x32x16(a, pp[i >> 2], acc[i & 3]);
    }
  };
  auto s_plain = [&](int ks, f32x16 (&sn)[2], bool use_pre) __attribute__((always_inline)) {
    int ksw[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) ksw[hf] = use_pre ? kswpre[hf] : read_ksw(ks, hf);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const i32x8 a = (t < NPK && use_pre) ? kpre[t < NPK ? t : 0] : read_k(ks, t);
      if (t < 2)
        sn[t & 1] = mfma_fp8<0, 0>(a, qf[0], negm, ksw[t & 1], qsw);
      else
        sn[t & 1] = mfma_fp8<2, 2>(a, qf[1], sn[t & 1], ksw[t & 1], qsw);
    }
  };
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
    const bool need_mask = (key0 + BN > n_keys) || (CAUSAL && key0 + BN - 1 > row0);
    if (need_mask) {
      const int lim = qlast;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = key0 + 16 * (r >> 3) + 8 * gq + (r & 7);
        if (kk > lim) sc[0][r] = -INFINITY;
        if (kk + 32 > lim) sc[1][r] = -INFINITY;
      }
    }
    const float sh = m2 == -INFINITY ? 0.f : m2;
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

  // ---- tile fetch: the DMA waves move K codes, K scales and V --------------
  // K codes: instruction i of DMA wave w fills key rows 8 (2w + i) .. +7 (1 KiB
  // of LDS); lane l writes physical chunk l & 7 of row 8 (2w + i) + (l >> 3)
  // and so fetches the logical chunk that the swizzle puts there.  K scales:
  // every DMA wave copies the tile's 64 scale words into its own copy (only
  // copy 0 is read), so that all DMA waves issue the same number of DMAs.
  // V: as the bf16 prefill (instruction i of wave w fills rows 16 i + 4 w ..).
  const bool dma_wave = wave < NDW;
  const int krs = p.Hkv * HD;          // bytes between K rows (e4m3)
  const int vrs = p.Hkv * HD * 2;      // bytes between V rows (bf16)
  int kb0, kb1, vb;
  {
    const int l8 = lane >> 3, pc = lane & 7;
    const int r0 = 16 * wave + l8, r1 = r0 + 8;
    kb0 = r0 * krs + 16 * k8_pos(r0, pc);
    kb1 = r1 * krs + 16 * k8_pos(r1, pc);
    const int r = 4 * wave + (lane >> 4), pos = lane & 15;
    vb = r * vrs + 16 * vd_pos(r, pos);
  }
  const int sb = lane * p.Hkv * 4;     // scale word of key row `lane`
  struct Stream {
    const char *base;   // first byte of the next tile
    int rows_left;      // key rows of this batch from there on
  };
  const size_t first = ((size_t)b * p.S) * p.Hkv + g;   // row index of key 0, head g
  Stream kst{static_cast<const char *>(p.k8) + first * HD, p.S};
  Stream sst{reinterpret_cast<const char *>(p.k_scale) + first * 4, p.S};
  Stream vst{static_cast<const char *>(p.v) + first * HD * 2, p.S};
  // the range of a tile ends at key row S of this batch (later rows read as
  // zero) or after the tile; tiles at or past n_tiles get an empty range
  auto range = [&](const Stream &st, int tile, int row_bytes) __attribute__((always_inline)) {
    const int nb = tile < n_tiles ? (min(st.rows_left, BN) * p.Hkv - g) * row_bytes : 0;
    return rsrc_words(st.base, nb);
  };
  auto issue_k = [&](int tile, int slot) __attribute__((always_inline)) {
    const u32x4 rk = range(kst, tile, HD);
    const u32x4 rsc = range(sst, tile, 4);
    char *dst = smem + slot + wave * 2048;
    dma_to_lds_16(rk, dst, opaque(kb0));
    dma_to_lds_16(rk, dst + 1024, opaque(kb1));
    dma_to_lds_4(rsc, smem + SBASE + (slot / KT) * ST + 256 * wave, opaque(sb));
    kst.base += (size_t)BN * krs;
    sst.base += (size_t)BN * p.Hkv * 4;
    kst.rows_left -= BN;
    sst.rows_left -= BN;
  };
  auto issue_v = [&](int tile, int slot) __attribute__((always_inline)) {
    const u32x4 rv = range(vst, tile, HD * 2);
    const int base = opaque(vb);
    char *dst = smem + slot + wave * 1024;
#pragma unroll
    for (int i = 0; i < VDPW; ++i) dma_to_lds_16(rv, dst + 4096 * i, base + i * 16 * vrs);
    vst.base += (size_t)BN * vrs;
    vst.rows_left -= BN;
  };

  // ---- prologue: K_0..K_{KA-1}, V_0..V_{VA-1} in flight, then S_0 --------
  if (dma_wave) {
#pragma unroll
    for (int t = 0; t < KA; ++t) issue_k(t, t * KT);
#pragma unroll
    for (int t = 0; t < VA; ++t) issue_v(t, VBASE + t * VT);
  }
  // K_0 and K_1 (codes and scales) first; the rest keeps landing during S_0
  wait_vmcnt<(KA - 2) * (KDPW + 1) + VA * VDPW>();
  barrier_no_wait();
  if (wave_tiles > 0) s_plain(0, S[0], false);   // K_0 in slot 0
  if (1 < wave_tiles) {
#pragma unroll
    for (int i = 0; i < NPK; ++i) kpre[i] = read_k(KT, i);
    kswpre[0] = read_ksw(KT, 0);
    kswpre[1] = read_ksw(KT, 1);
  }
  // iteration 0 reads operands of V_0 and K_2 before its own barrier, and
  // every DMA wave wrote part of them: publish all prologue tiles here
  wait_vmcnt<0>();
  barrier_no_wait();

  auto fetch = [&](int j, int kdst, int vdst) __attribute__((always_inline)) {
    if (dma_wave) {
      issue_k(j + KA, kdst);
      issue_v(j + VA, vdst);
    }
  };
  // End of iteration j: read the first operands of iteration j + 1; an even
  // j first waits for the DMAs of j - 1 (those of j may still fly) and ends
  // with the barrier that publishes them.
  auto finish = [&](int j, int v_next, int k_next2, bool pair_end) __attribute__((always_inline)) {
    if (pair_end) wait_vmcnt<DPI>();
    if (j < wave_tiles) {
#pragma unroll
      for (int i = 0; i < NPV; ++i) vpre[i] = read_v(v_next, i);
    }
    if (j + 2 < wave_tiles) {
#pragma unroll
      for (int i = 0; i < NPK; ++i) kpre[i] = read_k(k_next2, i);
      kswpre[0] = read_ksw(k_next2, 0);
      kswpre[1] = read_ksw(k_next2, 1);
    }
    if (pair_end) barrier_no_wait();
  };

  // Interleaved iteration j (j >= 1, j + 1 < wave_tiles, no mask).  Twenty
  // MFMA slots: 16 bf16 P V, then the 4 FP8 K Q^T.  The softmax of S_j runs
  // on 32 virtual slots (exp of score v in virtual slot v; pair pr = v / 2
  // packed to bf16 in slot 2pr + 2 and summed in 2pr + 3, as in the bf16
  // prefill); the P V slots carry virtual slots 0..15, one each, and each FP8
  // slot carries four of 16..31.
  auto fused = [&](int j, auto par_tag, auto ring_tag) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_tag)::value;
    constexpr int R = decltype(ring_tag)::value;
    f32x16 (&sc)[2] = S[PAR];
    f32x16 (&sn)[2] = S[PAR ^ 1];
    bf16x8 (&pc)[4] = P[PAR];
    const bf16x8 (&pp)[4] = P[PAR ^ 1];
    constexpr int kdma = ((R + KA) % NKS) * KT, ks = ((R + 1) % NKS) * KT,
                  kpre_s = ((R + 2) % NKS) * KT;
    constexpr int vdma = VBASE + ((R + VA) % NVS) * VT, vs = VBASE + ((R + NVS - 1) % NVS) * VT,
                  vpre_s = VBASE + R * VT;
    fetch(j, kdma, vdma);
    bf16x8 vop[16];
    i32x8 kop[4];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      vop[i] = vpre[i];
      kop[i] = kpre[i];
    }
    const int ksw0 = kswpre[0], ksw1 = kswpre[1];
    float ts = 0.f;
    float xs[2][2];
    auto valu = [&](auto v_tag) __attribute__((always_inline)) {
      constexpr int v = decltype(v_tag)::value;
      constexpr int pr = v >> 1;
      constexpr int hf = pr >> 3, r = 2 * (pr & 7) + (v & 1);
      xs[pr & 1][v & 1] = fast_exp2(sc[hf][r]);
      if constexpr (pr >= 1) {
        constexpr int q = pr - 1;
        if constexpr ((v & 1) == 0) {
          pc[q >> 2][2 * (q & 3)] = to_bf16(xs[q & 1][0]);
          pc[q >> 2][2 * (q & 3) + 1] = to_bf16(xs[q & 1][1]);
        } else {
          ts = add_bf16_pair(as_u32x4(pc[q >> 2])[q & 3], ts);
        }
      }
    };
    static_for<20>([&](auto slot_tag) __attribute__((always_inline)) {
      constexpr int i = decltype(slot_tag)::value;
      constexpr int nx = i + LA;   // operand read in this slot
      if constexpr (nx < 16)
        vop[nx] = read_v(vs, nx);
      else if constexpr (nx >= 16 + NPK && nx < 20)
        kop[nx - 16] = read_k(ks, nx - 16);
      if constexpr (i < 16) {
        acc[i & 3] = mfma_32x32x16(vop[i], pp[i >> 2], acc[i & 3]);
        valu(Int<i>{});
      } else {
        constexpr int t = i - 16;
        const int sw = (t & 1) ? ksw1 : ksw0;
        if constexpr (t < 2)
          sn[t & 1] = mfma_fp8<0, 0>(kop[t], qf[0], negm, sw, qsw);
        else
          sn[t & 1] = mfma_fp8<2, 2>(kop[t], qf[1], sn[t & 1], sw, qsw);
        valu(Int<16 + 4 * t>{});
        valu(Int<17 + 4 * t>{});
        valu(Int<18 + 4 * t>{});
        valu(Int<19 + 4 * t>{});
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    pc[3][6] = to_bf16(xs[1][0]);
    pc[3][7] = to_bf16(xs[1][1]);
    ts = add_bf16_pair(as_u32x4(pc[3])[3], ts);
#pragma unroll
    for (int u = 0; u < 4; ++u) asm volatile("" ::"v"(pc[u]));
    const float l_prev = l_run;
    l_run = l_prev + ts;
    asm volatile("" ::"v"(l_run));
    if (__ballot(!(ts <= kSumLimit))) {
      // rare: redo the tile against its exact maximum (see the bf16 prefill)
      const float dm = fmaxf(tile_max(sc), 0.f);
      const float alpha = fast_exp2(-dm);
      m2 += dm;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;
      l_run = exp_half(sc, pc, 1, dm, exp_half(sc, pc, 0, dm, l_prev * alpha));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sn[0][r] -= dm;
        sn[1][r] -= dm;
      }
      set_shift();
    }
    finish(j, vpre_s, kpre_s, R % 2 == 0);   // j = R (mod NKS), NKS even
  };

  // Plain iteration j: whatever of P_{j-1} V_{j-1}, softmax(S_j), S_{j+1}
  // this wave still has, one after the other (ring positions at run time).
  auto plain = [&](int j, auto par_tag) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_tag)::value;
    fetch(j, k_slot(j + KA), v_slot(j + VA));
    if (j >= 1 && j - 1 < wave_tiles) pv_plain(opaque(v_slot(j + NVS - 1)), P[PAR ^ 1]);   // V_{j-1}
    if (j < wave_tiles) softmax_plain(j, S[PAR], P[PAR]);
    if (j + 1 < wave_tiles) s_plain(opaque(k_slot(j + 1)), S[PAR ^ 1], true);
    finish(j, opaque(v_slot(j)), opaque(k_slot(j + 2)), (j & 1) == 0);
  };

  int fused_end = min(n_keys / BN, wave_tiles - 1);
  if (CAUSAL) fused_end = min(fused_end, (row0 + 1) / BN);
  plain(0, Int<0>{});
  int j = 1;
#pragma clang loop unroll(disable)
  for (; j + 5 < fused_end; j += 6) {
    fused(j, Int<1>{}, Int<1>{});
    fused(j + 1, Int<0>{}, Int<2>{});
    fused(j + 2, Int<1>{}, Int<3>{});
    fused(j + 3, Int<0>{}, Int<4>{});
    fused(j + 4, Int<1>{}, Int<5>{});
    fused(j + 5, Int<0>{}, Int<0>{});
  }
#pragma clang loop unroll(disable)
  for (; j <= n_tiles; j += 2) {
    plain(j, Int<1>{});
    if (j + 1 <= n_tiles) plain(j + 1, Int<0>{});
  }
  // an odd last iteration ends without a wait: let its DMAs land before the
  // workgroup's LDS is released
  wait_vmcnt<0>();

  // ---- epilogue: divide by l once, store O (bf16) and LSE ----------------
  const float l_tot = pair_sum32(l_run);
  if (qrow < p.S) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16 *op = static_cast<bf16 *>(p.o) + (((size_t)b * p.S + qrow) * p.Hq + h) * HD;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int hp = 0; hp < 2; ++hp) {
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const auto r = __builtin_amdgcn_permlane32_swap(
              __builtin_bit_cast(uint32_t, acc[db][4 * (2 * hp) + e] * inv),
              __builtin_bit_cast(uint32_t, acc[db][4 * (2 * hp + 1) + e] * inv), false, false);
          f[e] = __builtin_bit_cast(float, (uint32_t)r[0]);
          f[4 + e] = __builtin_bit_cast(float, (uint32_t)r[1]);
        }
        bf16x8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = to_bf16(f[e]);
        *reinterpret_cast<bf16x8 *>(op + 32 * db + 16 * hp + 8 * gq) = w;
      }
    }
    if (p.lse && gq == 0) {
      const float lse2 = l_tot > 0.f ? m2 + __log2f(l_tot) : -INFINITY;
      p.lse[((size_t)b * p.Hq + h) * p.S + qrow] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
    }
  }
}

}  // namespace

hipError_t launch_prefill_fp8(const PrefillFp8Params &p, hipStream_t stream) {
  const int group = p.Hq / p.Hkv;
  const int heads_per_wg = group >= NW ? NW : group;
  const int head_slices = group >= NW ? group / NW : 1;
  const int rows_wg = 32 * (NW / heads_per_wg);
  const int n_qblk = (p.S + rows_wg - 1) / rows_wg;
  const long long n_wg = (long long)n_qblk * p.B * p.Hkv * head_slices;
  if (n_wg <= 0) return hipSuccess;
  if (n_wg > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)n_wg), block(NT);
  if (p.causal)
    hipLaunchKernelGGL(prefill_fp8_kernel<true>, grid, block, 0, stream, p, heads_per_wg,
                       head_slices, n_qblk);
  else
    hipLaunchKernelGGL(prefill_fp8_kernel<false>, grid, block, 0, stream, p, heads_per_wg,
                       head_slices, n_qblk);
  return hipGetLastError();
}

}  // namespace lcat

// Tiled exact attention with both products on the FP8 (OCP e4m3) matrix
// cores of gfx950, head_dim 128.
//
// FA3's FP8 path ("Flash Attention and distributed inference", §18.5) runs
// S = Q K^T and O = P V on 8-bit operands with block quantisation.  S^T =
// K Q^T runs as in the FP8-score kernel (prefill_fp8.hip): per-32-dim E8M0
// scales on Q and K inside the scaled MFMA, the query multiplied by
// scale * log2(e) and quantised in the kernel (rotated first when rotation
// signs are given: incoherent processing, hadamard.h).  P V contracts over
// keys, so V's blocks run along keys: attn_quantize_fp8_v stores V^T
// (dimension-major) as e4m3 with one scale per (dim, 32 keys), and the
// weights are rounded to e4m3 in registers.  The weights are formed as
// P' = 2^(s - m + 3) (s, m in log2 units, m the running reference), which
// puts the weights near the row maximum in e4m3's normal range, and every P'
// stays at most 2^8.75 < 448: a tile whose weights would exceed it is
// rescaled to its exact maximum first.  The denominator l is the sum of the
// rounded weights themselves, formed by one more FP8 MFMA (16x16x128)
// against a 0/1 operand, so O = sum P' V / sum P' normalises exactly the
// weights that P V used.  The rest is the bf16 prefill: K/V tiles staged in
// LDS rings by DMA, S^T = K Q^T so that
// softmax statistics are lane-local, online softmax with a running maximum
// and denominator (§18.3), one division by l at the end (§18.4); scores never
// leave registers.
//
// Key order.  The lane that holds column q of S^T in half h receives keys
// 32 t + 16 h .. +15 of the S^T MFMA over key half t (K rows are read with
// bits 2 and 4 of the row index swapped), which is the order the P V MFMA
// wants for its B operand: bytes 0..15 keys 16 h .. +15 and bytes 16..31
// keys 32 + 16 h .. +15 of the 64-key tile.  Register i of the S^T MFMA
// then holds key 16 h + (i % 4) + 8 ((i / 4) % 2) + 4 (i / 8) of its half.
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
constexpr int KT = BN * HD;             // bytes of one e4m3 K tile [64 keys][128 dims]
constexpr int VT = HD * BN;             // bytes of one e4m3 V^T tile [128 dims][64 keys]
constexpr int ST = 1024;                // bytes of a scale slot (4 copies of 64 words)
constexpr int KA = 5;                   // iteration j fetches K_{j+KA}
constexpr int VA = 3;                   // iteration j fetches V_{j+VA}
constexpr int NKS = 6;                  // K (and K-scale) ring slots
constexpr int NVS = 6;                  // V (and V-scale) ring slots
constexpr int VBASE = NKS * KT;         // LDS byte offset of the V ring
constexpr int KSBASE = VBASE + NVS * VT;   // LDS byte offset of the K-scale ring
constexpr int VSBASE = KSBASE + NKS * ST;  // LDS byte offset of the V-scale ring
constexpr int LDS_BYTES = VSBASE + NVS * ST;
constexpr int LA = 2;                   // operands are read LA MFMA slots before their use
constexpr int NPV = LA;                 // P V operands read before the barrier
constexpr int NPK = 1;                  // K Q^T operands read before the barrier
constexpr int NDW = 4;                  // waves that issue the tile DMAs
constexpr int KDPW = KT / 1024 / NDW;   // code DMAs per DMA wave and K tile
constexpr int VDPW = VT / 1024 / NDW;   // code DMAs per DMA wave and V tile
constexpr int DPI = KDPW + 1 + VDPW + 1;   // DMAs per DMA wave and iteration
// Barriers come in pairs of iterations: only even iterations end with a DMA
// wait and a barrier.  A tile fetched in an odd iteration j is published at
// the end of j + 1, one fetched in an even iteration at the end of j + 2.
// K_i is first read at the end of iteration i - 2 (operands read ahead)
// and last read in iteration i - 1; V_i is first read at the end
// of iteration i and last read in iteration i + 1.  The fetch in iteration j
// follows the barrier of iteration j - 1 (j odd) or j - 2 (j even), and the
// slot it fills must have been read for the last time before that barrier.
static_assert(KA >= 5 && VA >= 3, "tiles are published before their first read");
static_assert(NKS >= KA + 1 && NVS >= VA + 3, "a slot is refilled after its last read");
static_assert(NKS == 6 && NVS == 6, "the interleaved loop is unrolled over a 6-slot ring");
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
static_assert(KDPW == 2 && VDPW == 2, "row mapping of the DMAs");

// P' = 2^(s - m + kPShift); weights are kept at most 2^kPMaxLog2 (< 448, the
// largest e4m3 value); an edge iteration rescales when the tile maximum
// exceeds the reference by more than kRescaleLog2 (P' <= 2^8 afterwards).
constexpr float kPShift = 3.0f;
constexpr float kPMaxLog2 = 8.75f;
constexpr float kRescaleLog2 = 5.0f;
constexpr int kFp8OneX4 = 0x38383838;   // four e4m3 ones

// l = column sums of P'^T on v_mfma_scale_f32_16x16x128_f8f6f4.  Its lane l
// covers row (A) or column (B) l % 16 and the K group l / 16, the same K
// elements in A and B; its result register r of lane l is row
// 4 (l / 16) + r, column l % 16.  P'^T as B: lane q + 32 h (q < 32) holds
// the 64 weights of query q split over the groups, so column j gathers
// queries j (groups 0, 2) and j + 16 (groups 1, 3).  The A operand selects
// groups 0, 2 for rows 0..3 and 8..11 and groups 1, 3 for rows 4..7 and
// 12..15: lane l then receives the sum of query l % 32 in every register.
// (That layout is the one of the 16x16 MFMA family; the uniform-V closed form
// in the tests, whose result depends on l alone, confirms it on the part.)
__device__ __forceinline__ i32x8 l_selector(int lane) {
  const int grp = lane >> 4, row = lane & 15;
  const int v = (grp & 1) == ((row >> 2) & 1) ? kFp8OneX4 : 0;
  return i32x8{v, v, v, v, v, v, v, v};
}
__device__ __forceinline__ f32x4 mfma_fp8_16(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, kE8m0OneX4, 0, kE8m0OneX4);
}

// e4m3 K tile: 64 key rows x 8 chunks of 16 dims (128-byte rows).  Chunk c
// of row r sits at c ^ f(r), f(r) = bit 1 of r | bits 3, 4 of r shifted to
// bits 1, 2: the 16 rows a quarter-wave reads for one operand chunk (bit 2
// fixed, the other four free) fall on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int k8_pos(int row, int c) { return c ^ (((row >> 1) & 1) | ((row >> 2) & 6)); }
// e4m3 V^T tile: 128 dim rows x 4 chunks of 16 keys (64-byte rows).  Chunk
// c of row d sits at c ^ ((d >> 2) & 3): the 16 consecutive rows of a
// quarter-wave's read fall on 16 distinct bank groups.
__device__ __forceinline__ int v8_pos(int d, int c) { return c ^ ((d >> 2) & 3); }

// Four values into one word of e4m3 codes (value i in byte i, nearest even),
// written over `old`: both half-words are replaced, and taking the register's
// previous contents as the merge source of the first one saves clearing it.
__device__ __forceinline__ int fp8x4_over(int old, float y0, float y1, float y2, float y3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, old, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, lo, true);
}

// Word w (0..3) of a key half of P'_j holds keys 16 h + 4 w .. +3, which
// sit in registers word_reg(w) .. +3 of the S^T MFMA over that half.
__device__ constexpr int word_reg(int w) { return w == 0 ? 0 : w == 1 ? 8 : w == 2 ? 4 : 12; }

// Schedule: iteration j interleaves
//   O^T += V_{j-1}^T P'_{j-1}^T  (4 scaled FP8 MFMA, operands from the V ring)
//   l   += sum P'_{j-1}          (1 FP8 MFMA against the 0/1 selector)
//   softmax of S_j -> P'_j       (VALU: 32 exp2, 16 e4m3 packs, 16 max3)
//   S_{j+1}^T = K_{j+1} Q^T      (4 scaled FP8 MFMA, operands from the K ring)
// and fetches K_{j+KA} (codes and scales) and V_{j+VA} (codes and scales).
template <bool CAUSAL>
__global__ __launch_bounds__(NT) void prefill_fp8pv_kernel(PrefillFp8PvParams p, int heads_per_wg,
                                                           int head_slices, int n_qblk, int s64) {
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
  // Rows past the end repeat the last row (finite data) and are never stored.
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
  // A row lr of the S^T MFMA over key half t is key row krow + 32 t, krow =
  // lr with bits 2 and 4 swapped.  K operand (t, c): chunks 4c + gq and
  // 4c + 2 + gq of that row.
  const int krow = (lr & ~20) | ((lr & 4) << 2) | ((lr & 16) >> 2);
  int kaddr[2][2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) kaddr[c][pt] = krow * 128 + 16 * k8_pos(krow, 4 * c + 2 * pt + gq);
  const int ksaddr = opaque(KSBASE + 4 * krow);   // K-scale word of key row krow, copy 0
  // V^T operand db: row 32 db + lr, chunks gq (keys 16 gq ..) and 2 + gq
  // (keys 32 + 16 gq ..); the swizzle does not depend on db.
  int va[2];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt) va[pt] = opaque(lr * 64 + 16 * v8_pos(lr, 2 * pt + gq));
  const int vsaddr = opaque(VSBASE + 4 * lane);   // V-scale word of this lane, copy 0

  auto read_v = [&](int vs, int db) __attribute__((always_inline)) -> i32x8 {
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(smem + vs + va[0] + 2048 * db);
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(smem + vs + va[1] + 2048 * db);
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto read_k = [&](int ks, int t) __attribute__((always_inline)) -> i32x8 {
    const int hf = t & 1, c = t >> 1;
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(smem + ks + kaddr[c][0] + 4096 * hf);
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(smem + ks + kaddr[c][1] + 4096 * hf);
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // K-scale word of half hf, shifted so that byte 2c holds block 2c + gq
  auto read_ksw = [&](int ks, int hf) __attribute__((always_inline)) -> int {
    const int w = *reinterpret_cast<const int *>(smem + ksaddr + (ks / KT) * ST + 128 * hf);
    return (int)((uint32_t)w >> (8 * gq));
  };
  // V-scale word: byte db = scale of dim 32 db + lr over keys 32 gq .. +31
  auto read_vsw = [&](int vs) __attribute__((always_inline)) -> int {
    return *reinterpret_cast<const int *>(smem + vsaddr + ((vs - VBASE) / VT) * ST);
  };
  // ring slots of K_t and V_t
  auto k_slot = [](int t) { return (int)((unsigned)t % NKS) * KT; };
  auto v_slot = [](int t) { return VBASE + (int)((unsigned)t % NVS) * VT; };

  const int qlast = CAUSAL ? min(n_keys - 1, qrow) : n_keys - 1;

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  f32x4 lacc = f32x4{};
  f32x16 S[2][2];
  i32x8 P[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    S[a][0] = S[a][1] = f32x16{};
    P[a] = i32x8{};
  }
  const i32x8 ones = l_selector(lane);
  i32x8 vpre[NPV];
  i32x8 kpre[NPK];
  int kswpre[2] = {0, 0};
  int vswpre = 0;
#pragma unroll
  for (int i = 0; i < NPV; ++i) vpre[i] = i32x8{};
#pragma unroll
  for (int i = 0; i < NPK; ++i) kpre[i] = i32x8{};
  float m2 = -INFINITY;   // running maximum (log2 units); P' = 2^(s - m2 + kPShift)
  f32x16 negm = f32x16{};
  auto set_shift = [&]() __attribute__((always_inline)) {
    const float sh = m2 == -INFINITY ? 0.f : kPShift - m2;
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = sh;
  };

  auto pack_all = [&](const f32x16 (&sc)[2], i32x8 &pc, float d) __attribute__((always_inline)) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int hf = w >> 2, r = word_reg(w & 3);
      pc[w] = fp8x4_over(pc[w], fast_exp2(sc[hf][r] - d), fast_exp2(sc[hf][r + 1] - d),
                         fast_exp2(sc[hf][r + 2] - d), fast_exp2(sc[hf][r + 3] - d));
    }
  };

  // ---- plain (sequential) pieces, used for edge iterations ----------------
  auto pv_plain = [&](int vs, const i32x8 &pp) __attribute__((always_inline)) {
    const int vsw = vswpre;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const i32x8 a = db < NPV ? vpre[db < NPV ? db : 0] : read_v(vs, db);
      if (db == 0) acc[0] = mfma_fp8<0, 0>(a, pp, acc[0], vsw, kE8m0OneX4);
      if (db == 1) acc[1] = mfma_fp8<1, 0>(a, pp, acc[1], vsw, kE8m0OneX4);
      if (db == 2) acc[2] = mfma_fp8<2, 0>(a, pp, acc[2], vsw, kE8m0OneX4);
      if (db == 3) acc[3] = mfma_fp8<3, 0>(a, pp, acc[3], vsw, kE8m0OneX4);
    }
    lacc = mfma_fp8_16(ones, pp, lacc);
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
  auto softmax_plain = [&](int t, f32x16 (&sc)[2], i32x8 &pc) __attribute__((always_inline)) {
    const int key0 = t * BN;
    const bool need_mask = (key0 + BN > n_keys) || (CAUSAL && key0 + BN - 1 > row0);
    if (need_mask) {
      const int lim = qlast;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = key0 + 16 * gq + (r & 3) + 8 * ((r >> 2) & 1) + 4 * (r >> 3);
        if (kk > lim) sc[0][r] = -INFINITY;
        if (kk + 32 > lim) sc[1][r] = -INFINITY;
      }
    }
    const float sh = m2 == -INFINITY ? 0.f : m2 - kPShift;   // sc = s - sh
    const float mx2 = tile_max(sc) + sh;
    const bool grow = mx2 > m2 + kRescaleLog2;
    if (__ballot(grow)) {
      const float m_new = grow ? mx2 : m2;
      const float alpha = grow ? fast_exp2(m2 - m_new) : 1.f;
      m2 = m_new;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;
      lacc *= alpha;
      set_shift();
    }
    const float d = m2 == -INFINITY ? 0.f : (m2 - kPShift) - sh;
    pack_all(sc, pc, d);
  };

  // ---- tile fetch: the DMA waves move K and V codes and scales -------------
  // K codes: instruction i of DMA wave w fills key rows 8 (2w + i) .. +7;
  // lane l writes physical chunk l & 7 of row 8 (2w + i) + (l >> 3).  V^T
  // codes: instruction i of wave w fills dim rows 16 (2w + i) .. +15; lane l
  // writes physical chunk l & 3 of row 16 (2w + i) + (l >> 2).  Scales: every
  // DMA wave copies the tile's 64 scale words into its own copy (only copy 0
  // is read), so that all DMA waves issue the same number of DMAs.
  const bool dma_wave = wave < NDW;
  const int krs = p.Hkv * HD;          // bytes between K rows (e4m3)
  int kb0, kb1, vb;
  {
    const int l8 = lane >> 3, pc = lane & 7;
    const int r0 = 16 * wave + l8, r1 = r0 + 8;
    kb0 = r0 * krs + 16 * k8_pos(r0, pc);
    kb1 = r1 * krs + 16 * k8_pos(r1, pc);
    const int d = 32 * wave + (lane >> 2);
    vb = d * s64 + 16 * v8_pos(d, lane & 3);
  }
  const int sb = lane * p.Hkv * 4;     // K-scale word of key row `lane`
  const int vb16 = vb + 16 * s64;      // second V^T code DMA: 16 dim rows further
  const int vsb = 4 * lane;            // V-scale word `lane`
  const size_t first = ((size_t)b * p.S) * p.Hkv + g;   // row index of key 0, head g
  const char *kbase = static_cast<const char *>(p.k8) + first * HD;
  const char *ksbase = reinterpret_cast<const char *>(p.k_scale) + first * 4;
  const size_t bg = (size_t)b * p.Hkv + g;
  const char *vbase = static_cast<const char *>(p.v8t) + bg * HD * s64;
  const char *vsbase = reinterpret_cast<const char *>(p.v_scale) + bg * (s64 / BN) * 256;
  int k_rows_left = p.S;
  // the range of a K tile ends at key row S of this batch (later rows read as
  // zero); V tiles are padded to 64 keys; tiles at or past n_tiles are empty
  auto issue_k = [&](int tile, int slot) __attribute__((always_inline)) {
    const bool live = tile < n_tiles;
    const int rows = min(k_rows_left, BN) * p.Hkv - g;
    const u32x4 rk = rsrc_words(kbase, live ? rows * HD : 0);
    const u32x4 rsc = rsrc_words(ksbase, live ? rows * 4 : 0);
    char *dst = smem + slot + wave * 2048;
    dma_to_lds_16(rk, dst, kb0);
    dma_to_lds_16(rk, dst + 1024, kb1);
    dma_to_lds_4(rsc, smem + KSBASE + (slot / KT) * ST + 256 * wave, sb);
    kbase += (size_t)BN * krs;
    ksbase += (size_t)BN * p.Hkv * 4;
    k_rows_left -= BN;
  };
  auto issue_v = [&](int tile, int slot) __attribute__((always_inline)) {
    const bool live = tile < n_tiles;
    const u32x4 rv = rsrc_words(vbase, live ? (HD - 1) * s64 + BN : 0);
    const u32x4 rvs = rsrc_words(vsbase, live ? 256 : 0);
    char *dst = smem + slot + wave * 2048;
    dma_to_lds_16(rv, dst, vb);
    dma_to_lds_16(rv, dst + 1024, vb16);
    dma_to_lds_4(rvs, smem + VSBASE + ((slot - VBASE) / VT) * ST + 256 * wave, vsb);
    vbase += BN;
    vsbase += 256;
  };

  // ---- prologue: K_0..K_{KA-1}, V_0..V_{VA-1} in flight, then S_0 --------
  if (dma_wave) {
#pragma unroll
    for (int t = 0; t < KA; ++t) issue_k(t, t * KT);
#pragma unroll
    for (int t = 0; t < VA; ++t) issue_v(t, VBASE + t * VT);
  }
  // K_0 and K_1 (codes and scales) first; the rest keeps landing during S_0
  wait_vmcnt<(KA - 2) * (KDPW + 1) + VA * (VDPW + 1)>();
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
      vswpre = read_vsw(v_next);
    }
    if (j + 2 < wave_tiles) {
#pragma unroll
      for (int i = 0; i < NPK; ++i) kpre[i] = read_k(k_next2, i);
      kswpre[0] = read_ksw(k_next2, 0);
      kswpre[1] = read_ksw(k_next2, 1);
    }
    if (pair_end) barrier_no_wait();
  };

  // Interleaved iteration j (j >= 1, j + 1 < wave_tiles, no mask).  Nine
  // MFMA slots: 4 P V, the l MFMA, 4 K Q^T.  Slot i < 8 computes the four
  // exponentials of word i of P'_j and folds them into the tile maximum; slot
  // i >= 1 packs word i - 1.  A tile whose maximum would give a weight above
  // 2^kPMaxLog2 is redone against its exact maximum afterwards.
  auto fused = [&](int j, auto par_tag, auto ring_tag) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_tag)::value;
    constexpr int R = decltype(ring_tag)::value;
    f32x16 (&sc)[2] = S[PAR];
    f32x16 (&sn)[2] = S[PAR ^ 1];
    i32x8 &pc = P[PAR];
    const i32x8 &pp = P[PAR ^ 1];
    constexpr int kdma = ((R + KA) % NKS) * KT, ks = ((R + 1) % NKS) * KT,
                  kpre_s = ((R + 2) % NKS) * KT;
    constexpr int vdma = VBASE + ((R + VA) % NVS) * VT, vs = VBASE + ((R + NVS - 1) % NVS) * VT,
                  vpre_s = VBASE + R * VT;
    fetch(j, kdma, vdma);
    i32x8 vop[4], kop[4];
#pragma unroll
    for (int i = 0; i < NPV; ++i) vop[i] = vpre[i];
#pragma unroll
    for (int i = 0; i < NPK; ++i) kop[i] = kpre[i];
    const int ksw0 = kswpre[0], ksw1 = kswpre[1], vsw = vswpre;
    float xs[2][4];
    float mx = 0.f;
    static_for<9>([&](auto slot_tag) __attribute__((always_inline)) {
      constexpr int i = decltype(slot_tag)::value;
      constexpr int nx = i + LA;   // operand read in this slot: V 0..3, none, K 5..8
      if constexpr (nx < 4) {
        if constexpr (nx >= NPV) vop[nx] = read_v(vs, nx);
      } else if constexpr (nx >= 5 + NPK && nx < 9) {
        kop[nx - 5] = read_k(ks, nx - 5);
      }
      if constexpr (i < 4) {
        acc[i] = mfma_fp8<i, 0>(vop[i], pp, acc[i], vsw, kE8m0OneX4);
      } else if constexpr (i == 4) {
        lacc = mfma_fp8_16(ones, pp, lacc);
      } else {
        constexpr int t = i - 5;
        const int sw = (t & 1) ? ksw1 : ksw0;
        if constexpr (t < 2)
          sn[t & 1] = mfma_fp8<0, 0>(kop[t], qf[0], negm, sw, qsw);
        else
          sn[t & 1] = mfma_fp8<2, 2>(kop[t], qf[1], sn[t & 1], sw, qsw);
      }
      if constexpr (i < 8) {
        constexpr int hf = i >> 2, r = word_reg(i & 3);
#pragma unroll
        for (int e = 0; e < 4; ++e) xs[i & 1][e] = fast_exp2(sc[hf][r + e]);
        if constexpr (i == 0)
          mx = max_raw(max3_raw(sc[hf][r], sc[hf][r + 1], sc[hf][r + 2]), sc[hf][r + 3]);
        else
          mx = max3_raw(max3_raw(mx, sc[hf][r], sc[hf][r + 1]), sc[hf][r + 2], sc[hf][r + 3]);
      }
      if constexpr (i >= 1) {
        constexpr int w = i - 1;
        pc[w] = fp8x4_over(pc[w], xs[w & 1][0], xs[w & 1][1], xs[w & 1][2], xs[w & 1][3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    asm volatile("" ::"v"(pc));
    if (__ballot(mx > kPMaxLog2)) {
      // rare: redo the tile against its exact maximum (P' <= 2^kPShift)
      const float dm = fmaxf(tile_max(sc) - kPShift, 0.f);
      const float alpha = fast_exp2(-dm);
      m2 += dm;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;
      lacc *= alpha;
      pack_all(sc, pc, dm);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sn[0][r] -= dm;
        sn[1][r] -= dm;
      }
      set_shift();
    }
    finish(j, vpre_s, kpre_s, R % 2 == 0);   // j = R (mod NKS), NKS even
  };

  // Plain iteration j: whatever of P'_{j-1} V_{j-1}, softmax(S_j), S_{j+1}
  // this wave still has, one after the other (ring positions at run time).
  auto plain = [&](int j, auto par_tag) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_tag)::value;
    fetch(j, k_slot(j + KA), v_slot(j + VA));
    if (j >= 1 && j - 1 < wave_tiles) pv_plain(v_slot(j + NVS - 1), P[PAR ^ 1]);   // V_{j-1}
    if (j < wave_tiles) softmax_plain(j, S[PAR], P[PAR]);
    if (j + 1 < wave_tiles) s_plain(k_slot(j + 1), S[PAR ^ 1], true);
    finish(j, v_slot(j), k_slot(j + 2), (j & 1) == 0);
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
  // every register of lacc holds the row's sum of P'
  const float l_tot = lacc[0];
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
      const float lse2 = l_tot > 0.f ? (m2 - kPShift) + __log2f(l_tot) : -INFINITY;
      p.lse[((size_t)b * p.Hq + h) * p.S + qrow] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
    }
  }
}

}  // namespace

hipError_t launch_prefill_fp8_pv(const PrefillFp8PvParams &p, hipStream_t stream) {
  const int group = p.Hq / p.Hkv;
  const int heads_per_wg = group >= NW ? NW : group;
  const int head_slices = group >= NW ? group / NW : 1;
  const int rows_wg = 32 * (NW / heads_per_wg);
  const int n_qblk = (p.S + rows_wg - 1) / rows_wg;
  const int s64 = (p.S + BN - 1) / BN * BN;
  const long long n_wg = (long long)n_qblk * p.B * p.Hkv * head_slices;
  if (n_wg <= 0) return hipSuccess;
  if (n_wg > 0x7FFFFFFFLL || (long long)HD * s64 > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)n_wg), block(NT);
  if (p.causal)
    hipLaunchKernelGGL(prefill_fp8pv_kernel<true>, grid, block, 0, stream, p, heads_per_wg,
                       head_slices, n_qblk, s64);
  else
    hipLaunchKernelGGL(prefill_fp8pv_kernel<false>, grid, block, 0, stream, p, heads_per_wg,
                       head_slices, n_qblk, s64);
  return hipGetLastError();
}

}  // namespace lcat

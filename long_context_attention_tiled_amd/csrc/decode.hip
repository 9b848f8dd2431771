// Single-token decode over the head-sharded paged KV cache, split over keys.
//
// Decode reads the whole cached history of each request once, so it is
// bound by HBM bandwidth: per-token decode time is the bytes read divided by
// the memory bandwidth ("Flash Attention and distributed inference", §18.12,
// the deployment case).  To spread one request's history over the whole GPU the key
// range is cut into splits; each split produces the unnormalised triple
// (m, l, O) of the online softmax (§18.3) and a second kernel merges the
// splits with the same rescale identity: M = max m_s, w_s = 2^(m_s - M),
// O = sum w_s O_s / sum w_s l_s.
//
// Pieces: by default the blocks of all requests and KV heads are laid end to
// end and shared out equally among 256 to 768 waves (stream_pieces), so a
// wave's share may span several (request, KV head) segments and a long and
// a short context load the GPU alike; with a fixed split size, one wave per
// (split, KV head, request).  Each piece writes one record per query head,
// and the merge kernel finds a segment's pieces arithmetically.
//
// Per block of a piece (decode_range):
//  * The GQA group of the KV head (up to 16 query heads) is the N axis of
//    v_mfma_f32_16x16x32_bf16; K rows are the M axis (S^T = K Q^T), so each
//    lane owns one query and its softmax statistics need only lane-local
//    work plus two exchanges.
//  * O^T = V^T P^T: V blocks are stored dimension-major, so the A operand
//    is a 16-byte read straight from HBM; the score registers already sit in
//    B-operand order because K rows are read in a fixed permuted order.
//  * K and V of a 64-token block go straight from HBM to registers; no LDS.
//  * Every 16-byte load instruction covers whole 128-byte lines: the lanes
//    of query slot qi < 8 fetch the first 64 bytes of a line, those of
//    qi + 8 the second 64 bytes of the same line, and one DPP move per word
//    (lane l and l ^ 8 of each 16-lane row) hands each lane the operand
//    the MFMA expects.  With that, the non-temporal hint pays: loads that
//    touched only half of each line ran 4% slower with it.
//  * Slots at or past ctx_len are excluded by index: scores are set to -inf
//    and their V entries to zero before any multiply (they may hold NaN).
//
// FP8 cache (OCP e4m3 with one fp32 scale per token for K and for V, the
// group-quantised cache of the Ulysses inference article, §5.4): the same
// loop reads 8 KiB K and V blocks, widens each 16-byte load to two bf16
// operands in registers (exact: every e4m3 value is a bf16 value),
// multiplies each score by its key's K scale and folds the V scale into P
// before P V.  Which head dims and keys a lane holds is relabelled so that
// one 16-byte load feeds two MFMA operands; Q is loaded in the same order.
#include "device.h"
#include "kernels.h"

namespace lcat {
namespace {

constexpr int HD = 128;
constexpr int BT = 64;
constexpr int REC = 132;   // floats per workspace record: O[128], m (log2 units), l, pad

// Loads that fill whole lines (see above) leave lane l of each 16-lane row
// (l = qi) holding, in `a`, the first half of a line of row r(qi & 7) when
// qi < 8 and its second half when qi >= 8, and in `b` the same halves of
// row r((qi & 7) + 8).  The operand of the first half for row r(qi) is then
// a (qi < 8) or b of lane qi - 8, and that of the second half a of lane
// qi + 8 or b (qi >= 8).  A row rotation by 8 lanes (DPP row_ror:8) reads
// lane qi ^ 8; the bank mask keeps the lanes that already hold their part.
constexpr int kDppRowRor8 = 0x128;
__device__ __forceinline__ u32x4 line_first_half(u32x4 a, u32x4 b) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)   // lanes 8..15 of each row (banks 2, 3) take b from lane ^ 8
    r[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)a[i], (int)b[i], kDppRowRor8, 0xF, 0xC, false);
  return r;
}
__device__ __forceinline__ u32x4 line_second_half(u32x4 a, u32x4 b) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)   // lanes 0..7 of each row (banks 0, 1) take a from lane ^ 8
    r[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)b[i], (int)a[i], kDppRowRor8, 0xF, 0x3, false);
  return r;
}

struct BlockRegs {
  u32x4 k[4][4];   // K of the four 16-key sub-tiles as loaded: [t][2h + x] = line h, rows x
  u32x4 v[2][8];   // V^T of eight 16-row d tiles as loaded: [x][dt] = rows x
};

constexpr int BLOCK_BYTES = BT * HD * 2;   // 16 KiB: one K block or one V block
constexpr int BLOCK_BYTES8 = BT * HD;     // 8 KiB: one fp8 K or V block

struct BlockRegs8 {
  u32x4 k[4][2];   // K of the four 16-key sub-tiles as loaded: [t][x] = rows x
  u32x4 v[8];      // V^T: eight 16-row d tiles, 16 keys each
  f32x4 ks[4];     // K scale of the keys whose scores land in s[t]
  f32x4 vs[4];     // V scale of the same keys
};

// Eight e4m3 values (two words) -> eight bf16 values, exactly.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Blocks j_begin .. j_begin+nblk-1 of (request b, KV head g), nblk >= 1;
// `tail` keys (1..64) are valid in the last one.  Writes the unnormalised
// (O, m, l) record of every query head of the group: head qi of the group at
// rec0 + qi * head_stride (floats).
template <bool FP8>
__device__ __forceinline__ void decode_range(const DecodeParams &p, int b, int g, int j_begin,
                                             int nblk, int tail, float *rec0,
                                             size_t head_stride) {
  const int lane = threadIdx.x;
  const int group = p.Hq / p.Hkv;
  const int qi = lane & 15;   // query (head within the group) owned by this lane
  const int g4 = lane >> 4;   // 8-wide K slice of the MFMA operands

  const bf16 *kp = static_cast<const bf16 *>(p.k_pool);
  const bf16 *vp = static_cast<const bf16 *>(p.v_pool);

  bf16x8 qf[4];
  {
    const int qh = g * group + min(qi, group - 1);   // padding lanes reuse a real head
    const bf16 *src = static_cast<const bf16 *>(p.q) + ((size_t)b * p.Hq + qh) * HD;
    // MFMA step s covers dims 32s + 8*g4 .. +7 (bf16 cache), or
    // 64*(s/2) + 16*g4 + 8*(s%2) .. +7 (fp8 cache: one 16-byte K load per two steps)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[s] = as_bf16x8(ld_global_16(src + (FP8 ? 64 * (s >> 1) + 16 * g4 + 8 * (s & 1)
                                                : 32 * s + 8 * g4)));
  }

  // Physical ids of this split's blocks, 64 per vector register (lane i holds
  // block i of the chunk); tags are checked for the whole chunk at once.  An
  // invalid id is reported and replaced by block 0 (rows undefined, no
  // out-of-range access).
  const int32_t *table = p.block_table + ((size_t)b * p.Hkv + g) * p.max_blocks;
  const int want = p.kv_head_base + g;
  auto load_ids = [&](int base) __attribute__((always_inline)) -> int {
    const bool in = base + lane < nblk;
    const int id = in ? table[j_begin + base + lane] : 0;
    const bool ok = id >= 0 && id < p.n_blocks;
    const int tag = ok ? p.block_head[id] : want;
    const unsigned long long bad_block = __ballot(in && !ok);
    const unsigned long long bad_tag = __ballot(in && ok && tag != want);
    if (p.dev_status && lane == 0 && (bad_block | bad_tag)) p.dev_status[0] = bad_block ? 2 : 1;
    return ok ? id : 0;
  };
  int ids = load_ids(0);
  int ids_base = 0;
  auto block_id = [&](int i) __attribute__((always_inline)) -> int {
    if (i - ids_base >= 64) {   // next chunk of 64 ids (only for splits over 4096 keys)
      ids_base += 64;
      ids = load_ids(ids_base);
    }
    return __builtin_amdgcn_readlane(ids, i - ids_base);
  };

  // K row (within a block) whose MFMA operand lane qi holds for sub-tile
  // t = 2w + e: r(qi) = 32w + 8*(qi>>2) + 4e + (qi&3); its score then lands
  // in register r of lane group g4 exactly where the B operand of P V
  // expects key 32w + 8*g4 + 4e + r.  d slice ds (dims 32 ds + 8 g4 ..) of
  // that row is half (ds & 1) of its 128-byte line ds >> 1.  Loads fill
  // whole lines: load x of line h brings rows r((qi & 7) + 8x), bytes
  // 128h + 64 (qi >> 3) + 16 g4; r(q + 8) = r(q) + 16.  V^T rows are head
  // dims, 128 bytes each: load x of d tile dt brings row 16 dt + (qi & 7) + 8x,
  // bytes 64 (qi >> 3) + 16 g4 (keys 32 (qi >> 3) + 8 g4 ..).
  const int k_voff = (8 * ((qi & 7) >> 2) + (qi & 3)) * (HD * 2) + 64 * (qi >> 3) + 16 * g4;
  const int v_voff = (qi & 7) * (BT * 2) + 64 * (qi >> 3) + 16 * g4;
  auto load_k = [&](BlockRegs &R, int blk) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(kp + (size_t)blk * BT * HD, BLOCK_BYTES);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int hx = 0; hx < 4; ++hx)   // hx = 2h + x
        R.k[t][hx] = buf_load_16_nt(r, k_voff + 128 * (hx >> 1) + 4096 * (hx & 1) + 1024 * (t & 1),
                                    8192 * (t >> 1));
  };
  auto load_v = [&](BlockRegs &R, int blk) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(vp + (size_t)blk * HD * BT, BLOCK_BYTES);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) R.v[x][dt] = buf_load_16_nt(r, v_voff + 1024 * x, 2048 * dt);
  };

  const float c2 = p.scale * kLog2e;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;

  // One 64-key block: S^T = K Q^T, online softmax, O^T += V^T P^T.  The
  // next block's K is requested as soon as this block's K registers are
  // consumed, its V as soon as the V registers are, so a full block of
  // loads is always in flight.  MASKED handles the final partial block.
  BlockRegs R;
  auto step = [&](auto masked_tag, int blk_next, bool has_next, int nv) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value != 0;
    f32x4 s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = f32x4{};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 a = R.k[t][2 * h], b = R.k[t][2 * h + 1];
        s[t] = mfma_16x16x32(as_bf16x8(line_first_half(a, b)), qf[2 * h], s[t]);
        s[t] = mfma_16x16x32(as_bf16x8(line_second_half(a, b)), qf[2 * h + 1], s[t]);
      }
    }
    if (has_next) load_k(R, blk_next);
    if constexpr (MASKED) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (32 * (t >> 1) + 8 * g4 + 4 * (t & 1) + r >= nv) s[t][r] = -INFINITY;
    }

    float mx = s[0][0];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[t][r]);
    mx = fmaxf(mx, wave_shfl_xor(mx, 16));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float msc = (m_new == -INFINITY) ? 0.f : m_new * c2;
    const float alpha = fast_exp2(m_run * c2 - msc);
    m_run = m_new;

    bf16x8 pb[2];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = fast_exp2(fmaf(s[t][r], c2, -msc));
        psum += pv;
        pb[t >> 1][4 * (t & 1) + r] = to_bf16(pv);
      }
    l_run = l_run * alpha + psum;
    // V^T operands: R.v[w][dt] = keys 32w + 8 g4 .. of head dim 16 dt + qi
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const u32x4 a = R.v[0][dt], b = R.v[1][dt];
      R.v[0][dt] = line_first_half(a, b);
      R.v[1][dt] = line_second_half(a, b);
    }
    if constexpr (MASKED) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k0 = 32 * w + 8 * g4 + 2 * e;
          const uint32_t keep = (k0 >= nv ? 0u : 0xFFFFu) | (k0 + 1 >= nv ? 0u : 0xFFFF0000u);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) R.v[w][dt][e] &= keep;
        }
      }
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      acc[dt] *= alpha;
#pragma unroll
      for (int w = 0; w < 2; ++w) acc[dt] = mfma_16x16x32(as_bf16x8(R.v[w][dt]), pb[w], acc[dt]);
    }
    if (has_next) load_v(R, blk_next);
  };

  if constexpr (!FP8) {
    int blk = block_id(0);
    load_k(R, blk);
    load_v(R, blk);
    for (int i = 0; i + 1 < nblk; ++i) {
      const int blk_next = block_id(i + 1);
      step(Int<0>{}, blk_next, true, BT);
    }
    if (tail == BT)
      step(Int<0>{}, 0, false, BT);
    else
      step(Int<1>{}, 0, false, tail);
  } else {
    // K row whose operand lane qi holds for sub-tile t: r(qi) =
    // 16*(qi>>2) + 4t + (qi&3); its score lands in register r of lane group
    // g4 as key 16*g4 + 4t + r, which is where the B operand of P V expects
    // it (V^T operand w of a lane holds keys 16*g4 + 8w .. +7).  Rows are
    // 128 bytes, one line: load x brings rows r((qi & 7) + 8x) = r(qi & 7) +
    // 32x, bytes 64 (qi >> 3) + 16 g4, and the operand of dims 64u + 16 g4 ..
    // is half u of the line.  V^T rows (64 bytes) are whole per 4 lanes.
    const uint8_t *kp8 = static_cast<const uint8_t *>(p.k_pool);
    const uint8_t *vp8 = static_cast<const uint8_t *>(p.v_pool);
    const int k8_voff = (16 * ((qi & 7) >> 2) + (qi & 3)) * HD + 64 * (qi >> 3) + 16 * g4;
    const int v8_voff = qi * BT + 16 * g4;
    const int sc_voff = 64 * g4;   // bytes: scales of keys 16*g4 ..
    BlockRegs8 R8;
    auto load_k8 = [&](int blk) __attribute__((always_inline)) {
      const __amdgpu_buffer_rsrc_t r = make_rsrc(kp8 + (size_t)blk * BLOCK_BYTES8, BLOCK_BYTES8);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int x = 0; x < 2; ++x) R8.k[t][x] = buf_load_16_nt(r, k8_voff + 4096 * x, 512 * t);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.k_scale + (size_t)blk * BT, BT * 4);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        R8.ks[t] = __builtin_bit_cast(f32x4, buf_load_16_nt(rs, sc_voff, 16 * t));
    };
    auto load_v8 = [&](int blk) __attribute__((always_inline)) {
      const __amdgpu_buffer_rsrc_t r = make_rsrc(vp8 + (size_t)blk * BLOCK_BYTES8, BLOCK_BYTES8);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) R8.v[dt] = buf_load_16_nt(r, v8_voff, 1024 * dt);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.v_scale + (size_t)blk * BT, BT * 4);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        R8.vs[t] = __builtin_bit_cast(f32x4, buf_load_16_nt(rs, sc_voff, 16 * t));
    };
    auto step8 = [&](auto masked_tag, int blk_next, bool has_next, int nv) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked_tag)::value != 0;
      f32x4 s[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        s[t] = f32x4{};
        const u32x4 kh[2] = {line_first_half(R8.k[t][0], R8.k[t][1]),
                             line_second_half(R8.k[t][0], R8.k[t][1])};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          s[t] = mfma_16x16x32(fp8x8_to_bf16(kh[u][0], kh[u][1]), qf[2 * u], s[t]);
          s[t] = mfma_16x16x32(fp8x8_to_bf16(kh[u][2], kh[u][3]), qf[2 * u + 1], s[t]);
        }
        s[t] *= R8.ks[t];
      }
      if (has_next) load_k8(blk_next);
      if constexpr (MASKED) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * g4 + 4 * t + r >= nv) s[t][r] = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {   // word e holds keys 16*g4 + 4e .. +3
          const int k0 = 16 * g4 + 4 * e;
          uint32_t keep = 0;
#pragma unroll
          for (int x = 0; x < 4; ++x) keep |= (k0 + x < nv ? 0xFFu : 0u) << (8 * x);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) R8.v[dt][e] &= keep;
        }
      }

      float mx = s[0][0];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[t][r]);
      mx = fmaxf(mx, wave_shfl_xor(mx, 16));
      mx = fmaxf(mx, wave_shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float msc = (m_new == -INFINITY) ? 0.f : m_new * c2;
      const float alpha = fast_exp2(m_run * c2 - msc);
      m_run = m_new;

      bf16x8 pb[2];
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pv = fast_exp2(fmaf(s[t][r], c2, -msc));
          psum += pv;
          float pw = pv * R8.vs[t][r];   // V scale folded into P
          if (MASKED && 16 * g4 + 4 * t + r >= nv) pw = 0.f;   // its scale may be anything
          pb[t >> 1][4 * (t & 1) + r] = to_bf16(pw);
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        acc[dt] *= alpha;
        acc[dt] = mfma_16x16x32(fp8x8_to_bf16(R8.v[dt][0], R8.v[dt][1]), pb[0], acc[dt]);
        acc[dt] = mfma_16x16x32(fp8x8_to_bf16(R8.v[dt][2], R8.v[dt][3]), pb[1], acc[dt]);
      }
      if (has_next) load_v8(blk_next);
    };
    int blk = block_id(0);
    load_k8(blk);
    load_v8(blk);
    for (int i = 0; i + 1 < nblk; ++i) {
      const int blk_next = block_id(i + 1);
      step8(Int<0>{}, blk_next, true, BT);
    }
    if (tail == BT)
      step8(Int<0>{}, 0, false, BT);
    else
      step8(Int<1>{}, 0, false, tail);
  }

  l_run += wave_shfl_xor(l_run, 16);
  l_run += wave_shfl_xor(l_run, 32);
  if (qi < group) {
    float *rec = rec0 + (size_t)qi * head_stride;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4 *>(rec + 16 * dt + 4 * g4) = acc[dt];
    if (g4 == 0) {
      rec[HD] = m_run == -INFINITY ? -INFINITY : m_run * c2;
      rec[HD + 1] = l_run;
    }
  }
}

template <bool FP8>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void decode_split_kernel(
    DecodeParams p) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  int ctx = p.ctx_len[b];
  if (ctx > p.max_blocks * BT) {   // longer than the block table: flag and clamp
    if (split == 0 && g == 0 && lane == 0 && p.dev_status) p.dev_status[0] = 2;
    ctx = p.max_blocks * BT;
  }
  const int t_begin = split * p.split_tokens;
  if (t_begin >= ctx) return;
  const int t_end = min(ctx, t_begin + p.split_tokens);
  const int nblk = (t_end - t_begin + BT - 1) / BT;
  const int tail = t_end - t_begin - (nblk - 1) * BT;   // keys in the last block (1..64)
  const int group = p.Hq / p.Hkv;
  decode_range<FP8>(p, b, g, t_begin / BT, nblk, tail,
               p.ws + (((size_t)b * p.Hq + g * group) * p.n_split + split) * REC,
               (size_t)p.n_split * REC);
}

// ---- stream split: equal shares of all (request, KV head, block) work -----
//
// The work of a launch is the sequence of segments s = b * Hkv + g (request
// b, KV head g), each of nblk(b) blocks, laid end to end: W units in all.
// Wave w of P takes units [w W / P, (w+1) W / P), which may start and end
// inside segments and cover several of them; for each segment piece it
// writes one record, at index w + s (pieces are ordered both by w and by s,
// so w + s numbers them without gaps or collisions).  Every wave gets the
// same number of blocks whatever the context lengths, so there is no tail of
// long splits, and no workgroup is launched for an empty key range.

// Blocks of request r: its context clamped to the block table, rounded up.
__device__ __forceinline__ int request_blocks(const DecodeParams &p, int r) {
  const int ctx = min(max(p.ctx_len[r], 0), p.max_blocks * BT);
  return (ctx + BT - 1) / BT;
}

__device__ __forceinline__ long long wave_scan_incl(long long v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

// Units before request `target` (target may be B) and in total.
__device__ __forceinline__ void unit_prefix(const DecodeParams &p, int target, long long &before,
                                            long long &total) {
  const int lane = threadIdx.x & 63;
  before = 0;
  total = 0;
  for (int c = 0; c < p.B; c += 64) {
    const int r = c + lane;
    const long long u = r < p.B ? (long long)p.Hkv * request_blocks(p, r) : 0;
    const long long incl = wave_scan_incl(u, lane);
    if (target >= c && target < c + 64)
      before = total + __shfl(incl - u, target - c, 64);   // exclusive sum at `target`
    total += __shfl(incl, 63, 64);
  }
  if (target >= p.B) before = total;
}

// Number of pieces the W units are cut into: about four blocks per wave at
// the least (whole multiples of 256 waves, so every XCD gets the same number),
// and at most `max_waves` (the launch).  Small steps (a few requests of a
// few thousand tokens) then have fewer, longer pieces and fewer records to
// merge: 4 requests x 8192 tokens ran 20.6 -> 16.4 us per call with 256
// waves instead of 768, while long mixes keep 768.
__device__ __forceinline__ long long stream_pieces(long long W, int max_waves) {
  const long long by_work = (W / (4 * 256)) * 256;
  return min((long long)max_waves, max(256LL, by_work));
}

// Request containing unit `pos` (< total) and the first unit of that request.
__device__ __forceinline__ void locate_unit(const DecodeParams &p, long long pos, int &req,
                                            long long &req_start) {
  const int lane = threadIdx.x & 63;
  long long off = 0;
  req = p.B - 1;
  req_start = 0;
  for (int c = 0; c < p.B; c += 64) {
    const int r = c + lane;
    const long long u = r < p.B ? (long long)p.Hkv * request_blocks(p, r) : 0;
    const long long incl = off + wave_scan_incl(u, lane);
    const unsigned long long hit = __ballot(r < p.B && incl > pos);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      req = c + l;
      req_start = __shfl(incl - u, l, 64);
      return;
    }
    off = __shfl(incl, 63, 64);
  }
}

template <bool FP8>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void decode_stream_kernel(
    DecodeParams p) {
  const int w = blockIdx.x, lane = threadIdx.x;
  if (w == 0 && p.dev_status) {   // contexts longer than the block table are flagged and clamped
    for (int r = lane; r < p.B; r += 64)
      if (p.ctx_len[r] > p.max_blocks * BT) p.dev_status[0] = 2;
  }
  long long before, W;
  unit_prefix(p, p.B, before, W);
  const long long P = stream_pieces(W, p.stream_waves);
  if (w >= P) return;
  const long long st = W * w / P, en = W * (w + 1) / P;
  if (st >= en) return;
  int b;
  long long req_start;
  locate_unit(p, st, b, req_start);
  const int group = p.Hq / p.Hkv;
  long long pos = st;
  while (pos < en && b < p.B) {
    const int nb = request_blocks(p, b);
    const long long req_end = req_start + (long long)p.Hkv * nb;
    if (pos >= req_end) {   // next request (skips empty ones)
      req_start = req_end;
      ++b;
      continue;
    }
    const long long off = pos - req_start;
    const int g = (int)(off / nb), blk = (int)(off - (long long)g * nb);
    const long long stop = min(en, req_start + (long long)(g + 1) * nb);
    const int n = (int)(stop - pos);
    const int ctx = min(max(p.ctx_len[b], 0), p.max_blocks * BT);
    const int tail = (blk + n == nb) ? ctx - (nb - 1) * BT : BT;
    const long long seg = (long long)b * p.Hkv + g;
    decode_range<FP8>(p, b, g, blk, n, tail, p.ws + (size_t)(w + seg) * group * REC, REC);
    pos = stop;
  }
}

// One workgroup (MERGE_WAVES waves) per (request, query head).  Wave w folds
// splits w, w + MERGE_WAVES, ... with lane l owning output channels 2l and
// 2l+1, then the waves' partial sums are combined through LDS.  Eight waves
// of eight pieces each take up to 64 pieces in one round of loads: short
// steps, whose (request, head) rows have tens of pieces, are bound by these
// rounds of dependent loads.
constexpr int MERGE_WAVES = 8;

// Merge of the records (pieces) of one (request, query head):
// O = sum w_i O_i / sum w_i l_i with w_i = 2^(m_i - M), M the largest piece
// maximum.  Each wave folds pieces wave, wave + MERGE_WAVES, ... in one
// pass, loading kMergeBatch pieces at a time and keeping its sums relative to
// the largest maximum it has seen (rescaled when that grows); the waves' sums
// are then brought to the common M and added.  `rec(i)` is the record of piece i
// (NULL: no record).
constexpr int kMergeBatch = 8;
template <class RecOf>
__device__ __forceinline__ void merge_records(const DecodeParams &p, int b, int h, int n_pieces,
                                              RecOf rec) {
  __shared__ float part[MERGE_WAVES][HD + 2];
  __shared__ float wmax[MERGE_WAVES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  bf16 *o = static_cast<bf16 *>(p.o) + ((size_t)b * p.Hq + h) * HD;

  float M = -INFINITY, n0 = 0.f, n1 = 0.f, den = 0.f;
  for (int s0 = wave; s0 < n_pieces; s0 += MERGE_WAVES * kMergeBatch) {
    float ms[kMergeBatch], ls[kMergeBatch];
    float2 ov[kMergeBatch];
#pragma unroll
    for (int c = 0; c < kMergeBatch; ++c) {
      const int s = s0 + c * MERGE_WAVES;
      const float *r = s < n_pieces ? rec(s) : nullptr;
      ms[c] = -INFINITY;
      ls[c] = 0.f;
      ov[c] = make_float2(0.f, 0.f);
      if (r) {
        ms[c] = r[HD];
        ls[c] = r[HD + 1];
        ov[c] = *reinterpret_cast<const float2 *>(r + 2 * lane);
      }
    }
    float bm = M;
#pragma unroll
    for (int c = 0; c < kMergeBatch; ++c) bm = fmaxf(bm, ms[c]);
    if (bm == -INFINITY) continue;
    const float a = M == -INFINITY ? 0.f : fast_exp2(M - bm);
    n0 *= a;
    n1 *= a;
    den *= a;
#pragma unroll
    for (int c = 0; c < kMergeBatch; ++c) {
      const float w = ms[c] == -INFINITY ? 0.f : fast_exp2(ms[c] - bm);
      n0 = fmaf(w, ov[c].x, n0);
      n1 = fmaf(w, ov[c].y, n1);
      den = fmaf(w, ls[c], den);
    }
    M = bm;
  }
  if (lane == 0) wmax[wave] = M;
  __syncthreads();
  float Mg = wmax[0];
#pragma unroll
  for (int w = 1; w < MERGE_WAVES; ++w) Mg = fmaxf(Mg, wmax[w]);
  const float a = M == -INFINITY ? 0.f : fast_exp2(M - Mg);
  part[wave][2 * lane] = n0 * a;
  part[wave][2 * lane + 1] = n1 * a;
  if (lane == 0) part[wave][HD] = den * a;
  __syncthreads();
  if (tid < HD) {
    float num = 0.f, dsum = 0.f;
#pragma unroll
    for (int w = 0; w < MERGE_WAVES; ++w) {
      num += part[w][tid];
      dsum += part[w][HD];
    }
    o[tid] = to_bf16(dsum > 0.f ? num / dsum : 0.f);
    if (p.lse && tid == 0)
      p.lse[(size_t)b * p.Hq + h] = dsum > 0.f ? (Mg + __log2f(dsum)) * kLn2 : -INFINITY;
  }
}

__device__ __forceinline__ void write_empty(const DecodeParams &p, int b, int h) {
  bf16 *o = static_cast<bf16 *>(p.o) + ((size_t)b * p.Hq + h) * HD;
  if (threadIdx.x < HD) o[threadIdx.x] = to_bf16(0.f);
  if (p.lse && threadIdx.x == 0) p.lse[(size_t)b * p.Hq + h] = -INFINITY;
}

// Fixed splits: records [b][h][split].
__global__ __launch_bounds__(64 * MERGE_WAVES) void decode_merge_kernel(DecodeParams p) {
  const int b = blockIdx.x / p.Hq, h = blockIdx.x % p.Hq;
  const int ctx = min(p.ctx_len[b], p.max_blocks * BT);
  if (ctx <= 0) {
    write_empty(p, b, h);
    return;
  }
  const int ns = (ctx + p.split_tokens - 1) / p.split_tokens;
  const float *rec = p.ws + ((size_t)b * p.Hq + h) * p.n_split * REC;
  merge_records(p, b, h, ns, [&](int s) -> const float * { return rec + (size_t)s * REC; });
}

// Stream split: the pieces of segment s = b * Hkv + g come from waves
// w_first .. w_last (those whose unit range meets the segment), record w + s.
__global__ __launch_bounds__(64 * MERGE_WAVES) void decode_merge_stream_kernel(DecodeParams p) {
  const int b = blockIdx.x / p.Hq, h = blockIdx.x % p.Hq;
  const int group = p.Hq / p.Hkv, g = h / group, qh = h - g * group;
  const int nb = request_blocks(p, b);
  if (nb == 0) {
    write_empty(p, b, h);
    return;
  }
  long long before, W;
  unit_prefix(p, b, before, W);
  const long long P = stream_pieces(W, p.stream_waves);
  const long long s0 = before + (long long)g * nb, s1 = s0 + nb;
  const long long w_first = ((s0 + 1) * P - 1) / W, w_last = (s1 * P - 1) / W;
  const long long seg = (long long)b * p.Hkv + g;
  merge_records(p, b, h, (int)(w_last - w_first + 1), [&](int i) -> const float * {
    const long long w = w_first + i;
    if (W * w / P == W * (w + 1) / P) return nullptr;   // wave with no units
    return p.ws + ((size_t)(w + seg) * group + qh) * REC;
  });
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream) {
  if (p.B <= 0) return hipSuccess;
  if (p.stream_waves > 0) {
    if (p.fp8)
      hipLaunchKernelGGL(decode_stream_kernel<true>, dim3(p.stream_waves), dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL(decode_stream_kernel<false>, dim3(p.stream_waves), dim3(64), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_stream_kernel, dim3(p.B * p.Hq), dim3(64 * MERGE_WAVES), 0,
                       stream, p);
    return hipGetLastError();
  }
  dim3 g1(p.n_split, p.Hkv, p.B), b1(64);
  if (p.fp8)
    hipLaunchKernelGGL(decode_split_kernel<true>, g1, b1, 0, stream, p);
  else
    hipLaunchKernelGGL(decode_split_kernel<false>, g1, b1, 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(p.B * p.Hq), b2(64 * MERGE_WAVES);
  hipLaunchKernelGGL(decode_merge_kernel, g2, b2, 0, stream, p);
  return hipGetLastError();
}

}  // namespace lcat

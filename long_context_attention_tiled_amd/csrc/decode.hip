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
// Split kernel, one wave per (split, KV head, request):
//  * The GQA group of the KV head (up to 16 query heads) is the N axis of
//    v_mfma_f32_16x16x32_bf16; K rows are the M axis (S^T = K Q^T), so each
//    lane owns one query and its softmax statistics need only lane-local
//    work plus two exchanges.
//  * O^T = V^T P^T: V blocks are stored dimension-major, so the A operand
//    is a 16-byte read straight from HBM; the score registers already sit in
//    B-operand order because K rows are read in a fixed permuted order.
//  * K and V of a 64-token block go straight from HBM to registers; no LDS.
//  * Slots at or past ctx_len are excluded by index: scores are set to -inf
//    and their V entries to zero before any multiply (they may hold NaN).
#include "device.h"
#include "kernels.h"

namespace lcat {
namespace {

constexpr int HD = 128;
constexpr int BT = 64;
constexpr int REC = 132;   // floats per workspace record: O[128], m (log2 units), l, pad

struct BlockRegs {
  u32x4 k[4][4];   // K rows of the four 16-key sub-tiles, four 32-wide d slices
  u32x4 v[2][8];   // V^T: two 32-key halves x eight 16-row d tiles
};

constexpr int BLOCK_BYTES = BT * HD * 2;   // 16 KiB: one K block or one V block

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
  const int j_begin = t_begin / BT;
  const int nblk = (t_end - t_begin + BT - 1) / BT;
  const int tail = t_end - t_begin - (nblk - 1) * BT;   // keys in the last block (1..64)
  const int group = p.Hq / p.Hkv;
  const int qi = lane & 15;   // query (head within the group) owned by this lane
  const int g4 = lane >> 4;   // 8-wide K slice of the MFMA operands

  const bf16 *kp = static_cast<const bf16 *>(p.k_pool);
  const bf16 *vp = static_cast<const bf16 *>(p.v_pool);

  bf16x8 qf[4];
  {
    const int qh = g * group + min(qi, group - 1);   // padding lanes reuse a real head
    const bf16 *src = static_cast<const bf16 *>(p.q) + ((size_t)b * p.Hq + qh) * HD + 8 * g4;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = as_bf16x8(ld_global_16(src + 32 * s));
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

  // K row (within a block) read by this lane for sub-tile t = 2w + e:
  //   32w + 8*(qi>>2) + 4e + (qi&3); its score then lands in register r of
  //   lane group g4 exactly where the B operand of P V expects key
  //   32w + 8*g4 + 4e + r.
  const int k_voff = (8 * (qi >> 2) + (qi & 3)) * (HD * 2) + 16 * g4;
  const int v_voff = qi * (BT * 2) + 16 * g4;
  auto load_k = [&](BlockRegs &R, int blk) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(kp + (size_t)blk * BT * HD, BLOCK_BYTES);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        R.k[t][s] = buf_load_16(r, k_voff + 64 * s + 1024 * (t & 1), 8192 * (t >> 1));
  };
  auto load_v = [&](BlockRegs &R, int blk) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(vp + (size_t)blk * HD * BT, BLOCK_BYTES);
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) R.v[w][dt] = buf_load_16(r, v_voff + 64 * w, 2048 * dt);
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
      for (int ds = 0; ds < 4; ++ds) s[t] = mfma_16x16x32(as_bf16x8(R.k[t][ds]), qf[ds], s[t]);
    }
    if (has_next) load_k(R, blk_next);
    if constexpr (MASKED) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (32 * (t >> 1) + 8 * g4 + 4 * (t & 1) + r >= nv) s[t][r] = -INFINITY;
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
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      acc[dt] *= alpha;
#pragma unroll
      for (int w = 0; w < 2; ++w) acc[dt] = mfma_16x16x32(as_bf16x8(R.v[w][dt]), pb[w], acc[dt]);
    }
    if (has_next) load_v(R, blk_next);
  };

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

  l_run += wave_shfl_xor(l_run, 16);
  l_run += wave_shfl_xor(l_run, 32);
  if (qi < group) {
    float *rec = p.ws + (((size_t)b * p.Hq + g * group + qi) * p.n_split + split) * REC;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4 *>(rec + 16 * dt + 4 * g4) = acc[dt];
    if (g4 == 0) {
      rec[HD] = m_run == -INFINITY ? -INFINITY : m_run * c2;
      rec[HD + 1] = l_run;
    }
  }
}

// One workgroup (4 waves) per (request, query head).  Wave w folds splits
// w, w+4, ... with lane l owning output channels 2l and 2l+1, then the four
// partial sums are combined through LDS.
constexpr int MERGE_WAVES = 4;

__global__ __launch_bounds__(64 * MERGE_WAVES) void decode_merge_kernel(DecodeParams p) {
  __shared__ float part[MERGE_WAVES][HD + 2];
  __shared__ float wmax[MERGE_WAVES];
  const int b = blockIdx.x / p.Hq, h = blockIdx.x % p.Hq;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ctx = min(p.ctx_len[b], p.max_blocks * BT);
  bf16 *o = static_cast<bf16 *>(p.o) + ((size_t)b * p.Hq + h) * HD;
  if (ctx <= 0) {
    if (tid < HD) o[tid] = to_bf16(0.f);
    if (p.lse && tid == 0) p.lse[(size_t)b * p.Hq + h] = -INFINITY;
    return;
  }
  const int ns = (ctx + p.split_tokens - 1) / p.split_tokens;
  const float *rec = p.ws + ((size_t)b * p.Hq + h) * p.n_split * REC;

  // global max of the split maxima
  float M = -INFINITY;
  for (int s = tid; s < ns; s += 64 * MERGE_WAVES) M = fmaxf(M, rec[(size_t)s * REC + HD]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, wave_shfl_xor(M, off));
  if (lane == 0) wmax[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));

  float n0 = 0.f, n1 = 0.f, den = 0.f;
  if (M != -INFINITY) {
#pragma unroll 4
    for (int s = wave; s < ns; s += MERGE_WAVES) {
      const float *r = rec + (size_t)s * REC;
      const float ms = r[HD];
      const float w = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
      const float2 ov = *reinterpret_cast<const float2 *>(r + 2 * lane);
      n0 = fmaf(w, ov.x, n0);
      n1 = fmaf(w, ov.y, n1);
      den = fmaf(w, r[HD + 1], den);
    }
  }
  part[wave][2 * lane] = n0;
  part[wave][2 * lane + 1] = n1;
  if (lane == 0) part[wave][HD] = den;
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
      p.lse[(size_t)b * p.Hq + h] = dsum > 0.f ? (M + __log2f(dsum)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream) {
  if (p.B <= 0) return hipSuccess;
  dim3 g1(p.n_split, p.Hkv, p.B), b1(64);
  hipLaunchKernelGGL(decode_split_kernel, g1, b1, 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(p.B * p.Hq), b2(64 * MERGE_WAVES);
  hipLaunchKernelGGL(decode_merge_kernel, g2, b2, 0, stream, p);
  return hipGetLastError();
}

}  // namespace lcat

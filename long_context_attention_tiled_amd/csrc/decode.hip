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

__global__ __launch_bounds__(64) void decode_split_kernel(DecodeParams p) {
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
  const int group = p.Hq / p.Hkv;
  const int qi = lane & 15;   // query (head within the group) owned by this lane
  const int g4 = lane >> 4;   // 8-wide K slice of the MFMA operands

  const bf16 *kp = static_cast<const bf16 *>(p.k_pool);
  const bf16 *vp = static_cast<const bf16 *>(p.v_pool);
  const u32x4 zero = {0u, 0u, 0u, 0u};

  bf16x8 qf[4];
  {
    const bool qv = qi < group;
    const bf16 *src = static_cast<const bf16 *>(p.q) + ((size_t)b * p.Hq + g * group + (qv ? qi : 0)) * HD + 8 * g4;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = as_bf16x8(qv ? ld_global_16(src + 32 * s) : zero);
  }

  // K row (within a block) read by this lane for sub-tile t = 2w + e:
  //   32w + 8*(qi>>2) + 4e + (qi&3); its score then lands in register r of
  //   the lane group 4*g4+r order used as the B operand of P V.
  const int krow_base = 8 * (qi >> 2) + (qi & 3);
  const float c2 = p.scale * kLog2e;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const int32_t *table = p.block_table + ((size_t)b * p.Hkv + g) * p.max_blocks;

  for (int t0 = t_begin; t0 < t_end; t0 += BT) {
    const int blk = table[t0 / BT];
    const bool ok = blk >= 0 && blk < p.n_blocks;
    if (!ok || p.block_head[blk] != p.kv_head_base + g) {
      if (lane == 0 && p.dev_status) p.dev_status[0] = ok ? 1 : 2;
      if (!ok) continue;
    }
    const int nv = min(BT, ctx - t0);
    const bf16 *kb = kp + (size_t)blk * BT * HD;
    const bf16 *vb = vp + (size_t)blk * HD * BT;

    u32x4 kr[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = 32 * (t >> 1) + 4 * (t & 1) + krow_base;
#pragma unroll
      for (int s = 0; s < 4; ++s) kr[t][s] = ld_global_16(kb + row * HD + 32 * s + 8 * g4);
    }
    u32x4 vr[2][8];
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) vr[w][dt] = ld_global_16(vb + (16 * dt + qi) * BT + 32 * w + 8 * g4);

    // S^T = K Q^T, four 16-key sub-tiles
    f32x4 s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = f32x4{};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) s[t] = mfma_16x16x32(as_bf16x8(kr[t][ds]), qf[ds], s[t]);
    }
    if (nv < BT) {
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
          for (int dt = 0; dt < 8; ++dt) vr[w][dt][e] &= keep;
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
        const float pv = fast_exp2(s[t][r] * c2 - msc);
        psum += pv;
        pb[t >> 1][4 * (t & 1) + r] = to_bf16(pv);
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      acc[dt] *= alpha;
#pragma unroll
      for (int w = 0; w < 2; ++w) acc[dt] = mfma_16x16x32(as_bf16x8(vr[w][dt]), pb[w], acc[dt]);
    }
  }

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

// One workgroup per (request, query head); thread d owns output channel d.
__global__ __launch_bounds__(HD) void decode_merge_kernel(DecodeParams p) {
  const int b = blockIdx.x / p.Hq, h = blockIdx.x % p.Hq;
  const int d = threadIdx.x;
  const int ctx = min(p.ctx_len[b], p.max_blocks * BT);
  bf16 *o = static_cast<bf16 *>(p.o) + ((size_t)b * p.Hq + h) * HD;
  if (ctx <= 0) {
    o[d] = to_bf16(0.f);
    if (p.lse && d == 0) p.lse[(size_t)b * p.Hq + h] = -INFINITY;
    return;
  }
  const int ns = (ctx + p.split_tokens - 1) / p.split_tokens;
  const float *rec = p.ws + ((size_t)b * p.Hq + h) * p.n_split * REC;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, rec[s * REC + HD]);
  float num = 0.f, den = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < ns; ++s) {
      const float ms = rec[s * REC + HD];
      if (ms == -INFINITY) continue;
      const float w = fast_exp2(ms - M);
      num = fmaf(w, rec[s * REC + d], num);
      den = fmaf(w, rec[s * REC + HD + 1], den);
    }
  }
  o[d] = to_bf16(den > 0.f ? num / den : 0.f);
  if (p.lse && d == 0) p.lse[(size_t)b * p.Hq + h] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream) {
  if (p.B <= 0) return hipSuccess;
  dim3 g1(p.n_split, p.Hkv, p.B), b1(64);
  hipLaunchKernelGGL(decode_split_kernel, g1, b1, 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(p.B * p.Hq), b2(HD);
  hipLaunchKernelGGL(decode_merge_kernel, g2, b2, 0, stream, p);
  return hipGetLastError();
}

}  // namespace lcat

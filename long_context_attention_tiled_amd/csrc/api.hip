// C-ABI entry points of libattn: argument validation, launch planning and
// dispatch.  Every check happens before the first HIP call, so an invalid
// call enqueues nothing.  The semantics of each entry point are documented
// in include/attn.h.
#include <stdint.h>

#include <mutex>

#include "../../include/attn.h"
#include "kernels.h"

#ifndef LCAT_BUILD_ID
#define LCAT_BUILD_ID "unknown"   // set by the build to the hash of the sources
#endif

namespace {

constexpr int kHeadDim = 128;
constexpr int kBlockTokens = 64;
constexpr int kDecodeRecord = 132;          // floats per decode split record
// split_tokens == 0: the key ranges of all requests are shared out equally
// among this many waves: three per CU of a 256-CU device, a multiple of the
// 8 XCDs.  Fewer concurrent streams read HBM faster here: 768 waves beat
// 2048 (two per SIMD) by 3% (bf16 cache) and 5% (fp8 cache); counts that do
// not split evenly over the XCDs (384, 640) are slower.
constexpr int kStreamWaves = 768;

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- fixed device scratch of attn_decode_noalloc ---------------------------
// The split records of the decode live in `scratch` (below); its device
// address is resolved once per device, with that device current, and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices];   // address of each device's copy, once resolved

}  // namespace

// One copy per GPU the library runs on, held until the process ends.  In host
// code this name is only a handle for hipGetSymbolAddress: kernels receive
// the address that call returns.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the device that runs `stream`.
int scratch_address(hipStream_t stream, void **out) {
  int dev = 0, cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return ATTN_ERR_HIP;
  if (stream) {
    hipDevice_t d = 0;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return ATTN_ERR_HIP;
    dev = d;
  } else {
    dev = cur;
  }
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return ATTN_ERR_HIP;
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr) return ATTN_ERR_HIP;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return ATTN_OK;
}

// No relayout output may overlap any input or another output.
bool qkv_disjoint(const void *const in[3], void *const out[3], const int H[3], int SP, int S_loc,
                  int D, int elem_bytes) {
  long long in_bytes[3], out_bytes[3];
  for (int t = 0; t < 3; ++t) {
    out_bytes[t] = (long long)SP * S_loc * (H[t] / SP) * D * elem_bytes;
    in_bytes[t] = (long long)SP * S_loc * H[t] * D * elem_bytes;
  }
  auto disjoint = [](const void *a, long long na, const void *b, long long nb) {
    const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
    return x + na <= y || y + nb <= x;
  };
  for (int t = 0; t < 3; ++t) {
    for (int u = 0; u < 3; ++u) {
      if (!disjoint(out[t], out_bytes[t], in[u], in_bytes[u])) return false;
      if (u != t && !disjoint(out[t], out_bytes[t], out[u], out_bytes[u])) return false;
    }
  }
  return true;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// GQA group sizes the bf16 kernels handle: divisors of 8 or multiples of 8.
// Host signs (128 values of +1 or -1, or NULL) -> the rotation's sign mask.
// Returns false when an entry is neither +1 nor -1.
inline bool hadamard_signs(const int8_t *signs, lcat::HadamardSigns &sg) {
  sg = lcat::HadamardSigns{};
  if (!signs) return true;
  for (int i = 0; i < 128; ++i) {
    if (signs[i] != 1 && signs[i] != -1) return false;
    if (signs[i] < 0) sg.neg[i >> 5] |= 1u << (i & 31);
  }
  sg.on = 1;
  return true;
}

inline bool group_ok(int Hq, int Hkv) {
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv) return false;
  const int g = Hq / Hkv;
  return (g <= 8 && 8 % g == 0) || (g % 8 == 0);
}

inline long long decode_n_split(int max_blocks, int split_tokens) {
  const long long keys = (long long)max_blocks * kBlockTokens;
  return (keys + split_tokens - 1) / split_tokens;
}

// Map of CP rank `rank` of N for a sequence of S tokens, or false if the
// split is not defined for these sizes.
bool cp_map(long long S, int N, int rank, int mode, lcat::CpMap &m, long long &n_tok) {
  if (S < 0 || N <= 0 || rank < 0 || rank >= N) return false;
  auto bound = [&](long long b, long long n) { return b * S / n; };
  m.start_b = 0;
  m.stride = 1;
  switch (mode) {
    case ATTN_CP_CONTIGUOUS:
      if (S < N) return false;
      m.start_a = bound(rank, N);
      m.len_a = bound(rank + 1, N) - m.start_a;
      n_tok = m.len_a;
      return true;
    case ATTN_CP_STRIPED:
      if (S % N) return false;
      m.start_a = rank;
      m.stride = N;
      m.len_a = S / N;
      n_tok = m.len_a;
      return true;
    case ATTN_CP_ZIGZAG: {
      if (S < 2LL * N) return false;
      const long long a = rank, b = 2LL * N - 1 - rank;
      m.start_a = bound(a, 2LL * N);
      m.len_a = bound(a + 1, 2LL * N) - m.start_a;
      m.start_b = bound(b, 2LL * N);
      n_tok = m.len_a + (bound(b + 1, 2LL * N) - m.start_b);
      return true;
    }
    default:
      return false;
  }
}

// Argument checks, then the workspace: `get_ws(need, &ptr)` points ptr
// at a buffer for `need` bytes of split records, or returns an error status.
template <class GetWs>
int decode_common(const void *q, const void *k_pool, const void *v_pool, const float *k_scale,
                  const float *v_scale, int fp8, int n_blocks, const int32_t *block_head,
                  const int32_t *block_table, int max_blocks, const int32_t *ctx_len, void *o,
                  float *lse, int B, int Hq, int Hkv, int D, int kv_head_base, float scale,
                  int split_tokens, GetWs get_ws, int32_t *dev_status, void *stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || n_blocks <= 0 || max_blocks <= 0)
    return ATTN_ERR_SHAPE;
  if (split_tokens < 0 || split_tokens % kBlockTokens) return ATTN_ERR_SHAPE;
  if (D != kHeadDim || Hq / Hkv > 16) return ATTN_ERR_UNSUPPORTED;
  if (B == 0) return ATTN_OK;
  if (!q || !k_pool || !v_pool || !block_head || !block_table || !ctx_len || !o)
    return ATTN_ERR_NULL;
  if (fp8 && (!k_scale || !v_scale)) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool)) return ATTN_ERR_ALIGN;
  if (fp8 && (!aligned16(k_scale) || !aligned16(v_scale))) return ATTN_ERR_ALIGN;
  const size_t need = attn_decode_workspace_bytes(B, Hq, D, max_blocks, split_tokens);
  void *workspace = nullptr;
  const int ws_status = get_ws(need, &workspace);
  if (ws_status != ATTN_OK) return ws_status;
  const long long n_split = split_tokens ? decode_n_split(max_blocks, split_tokens) : 0;
  if (n_split > 0x7FFFFFFFLL) return ATTN_ERR_UNSUPPORTED;
  lcat::DecodeParams p{};
  p.q = q; p.k_pool = k_pool; p.v_pool = v_pool;
  p.k_scale = k_scale; p.v_scale = v_scale; p.fp8 = fp8;
  p.block_head = block_head; p.block_table = block_table; p.ctx_len = ctx_len;
  p.o = o; p.lse = lse; p.ws = static_cast<float *>(workspace); p.dev_status = dev_status;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.max_blocks = max_blocks; p.n_blocks = n_blocks;
  p.kv_head_base = kv_head_base; p.split_tokens = split_tokens; p.n_split = (int)n_split;
  p.stream_waves = split_tokens ? 0 : kStreamWaves;
  p.scale = scale;
  return hip_status(lcat::launch_decode(p, static_cast<hipStream_t>(stream)));
}

// The caller's workspace: at least `need` bytes, 16-byte aligned.
struct CallerWorkspace {
  void *ptr;
  size_t bytes;
  int operator()(size_t need, void **out) const {
    if (!ptr || bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned16(ptr)) return ATTN_ERR_ALIGN;
    *out = ptr;
    return ATTN_OK;
  }
};

}  // namespace

extern "C" {

const char *attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape or rank";
    case ATTN_ERR_DTYPE: return "unsupported dtype or element size";
    case ATTN_ERR_ALIGN: return "pointer not 16-byte aligned";
    case ATTN_ERR_UNSUPPORTED: return "configuration not supported";
    case ATTN_ERR_WORKSPACE: return "decode workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
    case ATTN_ERR_SCRATCH:
      return "call needs more decode scratch than the fixed device array of attn_decode_noalloc holds";
    default: return "unknown status";
  }
}

const char *attn_build_id(void) { return LCAT_BUILD_ID; }

int attn_prefill(const void *q, const void *k, const void *v, void *o, float *lse, int B, int S,
                 int Hq, int Hkv, int D, int dtype, int causal, float scale, void *stream) {
  if (B < 0 || S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_DTYPE;
  if (B == 0 || S == 0) return ATTN_OK;
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == ATTN_DTYPE_F32) {
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_ALIGN;
    return hip_status(lcat::launch_attn_f32(static_cast<const float *>(q),
                                            static_cast<const float *>(k),
                                            static_cast<const float *>(v), static_cast<float *>(o),
                                            lse, B, S, Hq, Hkv, D, causal, scale, st));
  }
  if (D != kHeadDim || !group_ok(Hq, Hkv)) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_ALIGN;
  lcat::PrefillParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.Sq = S; p.Sk = S; p.Hq = Hq; p.Hkv = Hkv;
  p.causal = causal != 0;
  p.scale = scale;
  return hip_status(lcat::launch_prefill_bf16(p, false, st));
}

int attn_quantize_fp8_blocks(const void *x, void *codes, uint8_t *scales, long long rows, int D,
                             const int8_t *signs, void *stream) {
  if (rows < 0 || D <= 0) return ATTN_ERR_SHAPE;
  if (D % 32 || (signs && D != kHeadDim)) return ATTN_ERR_UNSUPPORTED;
  lcat::HadamardSigns sg;
  if (!hadamard_signs(signs, sg)) return ATTN_ERR_SHAPE;
  if (rows == 0) return ATTN_OK;
  if (!x || !codes || !scales) return ATTN_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes)) return ATTN_ERR_ALIGN;
  const long long n = rows * D;
  auto overlap = [](const void *a, long long na, const void *b, long long nb) {
    const char *x0 = static_cast<const char *>(a), *y0 = static_cast<const char *>(b);
    return x0 < y0 + nb && y0 < x0 + na;
  };
  if (overlap(x, 2 * n, codes, n) || overlap(x, 2 * n, scales, n / 32) ||
      overlap(codes, n, scales, n / 32))
    return ATTN_ERR_SHAPE;
  if (sg.on)
    return hip_status(lcat::launch_quantize_fp8_rotated(x, codes, scales, rows, sg,
                                                        static_cast<hipStream_t>(stream)));
  return hip_status(lcat::launch_quantize_fp8_blocks(x, codes, scales, n / 32,
                                                     static_cast<hipStream_t>(stream)));
}

int attn_prefill_fp8(const void *q, const void *k8, const uint8_t *k_scale, const void *v, void *o,
                     float *lse, int B, int S, int Hq, int Hkv, int D, int causal, float scale,
                     const int8_t *signs, void *stream) {
  if (B < 0 || S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return ATTN_ERR_SHAPE;
  if (D != kHeadDim || !group_ok(Hq, Hkv)) return ATTN_ERR_UNSUPPORTED;
  lcat::HadamardSigns sg;
  if (!hadamard_signs(signs, sg)) return ATTN_ERR_SHAPE;
  if (B == 0 || S == 0) return ATTN_OK;
  if (!q || !k8 || !k_scale || !v || !o) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k8) || !aligned16(v) || !aligned16(o) ||
      reinterpret_cast<uintptr_t>(k_scale) % 4)
    return ATTN_ERR_ALIGN;
  lcat::PrefillFp8Params p{};
  p.q = q; p.k8 = k8; p.k_scale = k_scale; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.S = S; p.Hq = Hq; p.Hkv = Hkv;
  p.causal = causal != 0;
  p.scale = scale;
  p.rot = sg;
  return hip_status(lcat::launch_prefill_fp8(p, static_cast<hipStream_t>(stream)));
}

int attn_quantize_fp8_v(const void *v, void *v8t, uint8_t *v_scale, int B, int S, int Hkv, int D,
                        void *stream) {
  if (B < 0 || S < 0 || Hkv <= 0 || D <= 0) return ATTN_ERR_SHAPE;
  if (D != kHeadDim) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || S == 0) return ATTN_OK;
  if (!v || !v8t || !v_scale) return ATTN_ERR_NULL;
  if (!aligned16(v) || !aligned16(v8t)) return ATTN_ERR_ALIGN;
  const long long s64 = ((long long)S + 63) / 64 * 64;
  const long long nv = (long long)B * S * Hkv * D * 2;
  const long long n8 = (long long)B * Hkv * D * s64;
  const long long ns = (long long)B * Hkv * (s64 / 64) * 256;
  if (D * s64 > 0x7FFFFFFFLL) return ATTN_ERR_SHAPE;
  auto overlap = [](const void *a, long long na, const void *b, long long nb) {
    const char *x0 = static_cast<const char *>(a), *y0 = static_cast<const char *>(b);
    return x0 < y0 + nb && y0 < x0 + na;
  };
  if (overlap(v, nv, v8t, n8) || overlap(v, nv, v_scale, ns) || overlap(v8t, n8, v_scale, ns))
    return ATTN_ERR_SHAPE;
  return hip_status(lcat::launch_quantize_fp8_v(v, v8t, v_scale, B, S, Hkv,
                                                static_cast<hipStream_t>(stream)));
}

int attn_prefill_fp8_pv(const void *q, const void *k8, const uint8_t *k_scale, const void *v8t,
                        const uint8_t *v_scale, void *o, float *lse, int B, int S, int Hq, int Hkv,
                        int D, int causal, float scale, const int8_t *signs, void *stream) {
  if (B < 0 || S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return ATTN_ERR_SHAPE;
  if (D != kHeadDim || !group_ok(Hq, Hkv)) return ATTN_ERR_UNSUPPORTED;
  lcat::HadamardSigns sg;
  if (!hadamard_signs(signs, sg)) return ATTN_ERR_SHAPE;
  if (B == 0 || S == 0) return ATTN_OK;
  if ((long long)D * (((long long)S + 63) / 64 * 64) > 0x7FFFFFFFLL) return ATTN_ERR_SHAPE;
  if (!q || !k8 || !k_scale || !v8t || !v_scale || !o) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k8) || !aligned16(v8t) || !aligned16(o) ||
      reinterpret_cast<uintptr_t>(k_scale) % 4 || reinterpret_cast<uintptr_t>(v_scale) % 4)
    return ATTN_ERR_ALIGN;
  lcat::PrefillFp8PvParams p{};
  p.q = q; p.k8 = k8; p.k_scale = k_scale; p.v8t = v8t; p.v_scale = v_scale; p.o = o; p.lse = lse;
  p.B = B; p.S = S; p.Hq = Hq; p.Hkv = Hkv;
  p.causal = causal != 0;
  p.scale = scale;
  p.rot = sg;
  return hip_status(lcat::launch_prefill_fp8_pv(p, static_cast<hipStream_t>(stream)));
}

int attn_kv_append(const void *k_new, const void *v_new, void *k_pool, void *v_pool, int n_blocks,
                   const int32_t *block_head, const int32_t *block_table, int max_blocks,
                   const int32_t *start_pos, int T, int B, int Hkv, int D, int kv_head_base,
                   int32_t *dev_status, void *stream) {
  if (T < 0 || B < 0 || Hkv <= 0 || n_blocks <= 0 || max_blocks <= 0) return ATTN_ERR_SHAPE;
  if (D != kHeadDim) return ATTN_ERR_UNSUPPORTED;
  if (T == 0 || B == 0) return ATTN_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_head || !block_table || !start_pos)
    return ATTN_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return ATTN_ERR_ALIGN;
  return hip_status(lcat::launch_kv_append(k_new, v_new, k_pool, v_pool, n_blocks, block_head,
                                           block_table, max_blocks, start_pos, T, B, Hkv,
                                           kv_head_base, dev_status,
                                           static_cast<hipStream_t>(stream)));
}

int attn_chunked_prefill(const void *q, const void *k_new, const void *v_new, void *k_pool,
                         void *v_pool, int n_blocks, const int32_t *block_head,
                         const int32_t *block_table, int max_blocks, const int32_t *ctx_before,
                         int C, void *o, float *lse, int B, int Hq, int Hkv, int D,
                         int kv_head_base, float scale, int32_t *dev_status, void *stream) {
  if (C < 0 || B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || n_blocks <= 0 || max_blocks <= 0)
    return ATTN_ERR_SHAPE;
  if (D != kHeadDim || !group_ok(Hq, Hkv)) return ATTN_ERR_UNSUPPORTED;
  if (C == 0 || B == 0) return ATTN_OK;
  if (!q || !k_new || !v_new || !k_pool || !v_pool || !block_head || !block_table || !ctx_before ||
      !o)
    return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) ||
      !aligned16(v_pool) || !aligned16(o))
    return ATTN_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int rc = hip_status(lcat::launch_kv_append(k_new, v_new, k_pool, v_pool, n_blocks, block_head,
                                             block_table, max_blocks, ctx_before, C, B, Hkv,
                                             kv_head_base, dev_status, st));
  if (rc != ATTN_OK) return rc;
  lcat::PrefillParams p{};
  p.q = q; p.k = k_pool; p.v = v_pool; p.o = o; p.lse = lse;
  p.block_table = block_table; p.block_head = block_head; p.ctx_before = ctx_before;
  p.dev_status = dev_status;
  p.B = B; p.Sq = C; p.Sk = 0; p.Hq = Hq; p.Hkv = Hkv;
  p.max_blocks = max_blocks; p.n_blocks = n_blocks; p.kv_head_base = kv_head_base;
  p.causal = 1;
  p.scale = scale;
  return hip_status(lcat::launch_prefill_bf16(p, true, st));
}

size_t attn_decode_workspace_bytes(int B, int Hq, int D, int max_blocks, int split_tokens) {
  if (B < 0 || Hq <= 0 || D != kHeadDim || max_blocks <= 0 || split_tokens < 0 ||
      split_tokens % kBlockTokens)
    return 0;
  if (split_tokens == 0)   // at most kStreamWaves + B*Hkv pieces of group records
    return ((size_t)kStreamWaves + B) * Hq * kDecodeRecord * sizeof(float);
  return (size_t)B * Hq * decode_n_split(max_blocks, split_tokens) * kDecodeRecord * sizeof(float);
}

int attn_decode(const void *q, const void *k_pool, const void *v_pool, int n_blocks,
                const int32_t *block_head, const int32_t *block_table, int max_blocks,
                const int32_t *ctx_len, void *o, float *lse, int B, int Hq, int Hkv, int D,
                int kv_head_base, float scale, int split_tokens, void *workspace,
                size_t workspace_bytes, int32_t *dev_status, void *stream) {
  return decode_common(q, k_pool, v_pool, nullptr, nullptr, 0, n_blocks, block_head, block_table,
                       max_blocks, ctx_len, o, lse, B, Hq, Hkv, D, kv_head_base, scale,
                       split_tokens, CallerWorkspace{workspace, workspace_bytes}, dev_status,
                       stream);
}

int attn_decode_noalloc(const void *q, const void *k_pool, const void *v_pool, int n_blocks,
                        const int32_t *block_head, const int32_t *block_table, int max_blocks,
                        const int32_t *ctx_len, void *o, float *lse, int B, int Hq, int Hkv, int D,
                        int kv_head_base, float scale, int split_tokens, int32_t *dev_status,
                        void *stream) {
  // The records go to this device's `scratch`: no allocation, and nothing
  // in it needs clearing (the merge reads only records this call writes).
  auto fixed_scratch = [stream](size_t need, void **out) -> int {
    if (need > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
    return scratch_address(static_cast<hipStream_t>(stream), out);
  };
  return decode_common(q, k_pool, v_pool, nullptr, nullptr, 0, n_blocks, block_head, block_table,
                       max_blocks, ctx_len, o, lse, B, Hq, Hkv, D, kv_head_base, scale,
                       split_tokens, fixed_scratch, dev_status, stream);
}

int attn_decode_fp8(const void *q, const void *k8_pool, const void *v8_pool, const float *k_scale,
                    const float *v_scale, int n_blocks, const int32_t *block_head,
                    const int32_t *block_table, int max_blocks, const int32_t *ctx_len, void *o,
                    float *lse, int B, int Hq, int Hkv, int D, int kv_head_base, float scale,
                    int split_tokens, void *workspace, size_t workspace_bytes,
                    int32_t *dev_status, void *stream) {
  return decode_common(q, k8_pool, v8_pool, k_scale, v_scale, 1, n_blocks, block_head,
                       block_table, max_blocks, ctx_len, o, lse, B, Hq, Hkv, D, kv_head_base,
                       scale, split_tokens, CallerWorkspace{workspace, workspace_bytes},
                       dev_status, stream);
}

int attn_kv_append_fp8(const void *k_new, const void *v_new, void *k8_pool, void *v8_pool,
                       float *k_scale, float *v_scale, int n_blocks, const int32_t *block_head,
                       const int32_t *block_table, int max_blocks, const int32_t *start_pos, int T,
                       int B, int Hkv, int D, int kv_head_base, int32_t *dev_status,
                       void *stream) {
  if (T < 0 || B < 0 || Hkv <= 0 || n_blocks <= 0 || max_blocks <= 0) return ATTN_ERR_SHAPE;
  if (D != kHeadDim) return ATTN_ERR_UNSUPPORTED;
  if (T == 0 || B == 0) return ATTN_OK;
  if (!k_new || !v_new || !k8_pool || !v8_pool || !k_scale || !v_scale || !block_head ||
      !block_table || !start_pos)
    return ATTN_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k8_pool) || !aligned16(v8_pool))
    return ATTN_ERR_ALIGN;
  return hip_status(lcat::launch_kv_append_fp8(k_new, v_new, k8_pool, v8_pool, k_scale, v_scale,
                                               n_blocks, block_head, block_table, max_blocks,
                                               start_pos, T, B, Hkv, kv_head_base, dev_status,
                                               static_cast<hipStream_t>(stream)));
}

int attn_kv_quantize_fp8(const void *k_pool, const void *v_pool, void *k8_pool, void *v8_pool,
                         float *k_scale, float *v_scale, int n_blocks, int D, void *stream) {
  if (n_blocks < 0) return ATTN_ERR_SHAPE;
  if (D != kHeadDim) return ATTN_ERR_UNSUPPORTED;
  if (n_blocks == 0) return ATTN_OK;
  if (!k_pool || !v_pool || !k8_pool || !v8_pool || !k_scale || !v_scale) return ATTN_ERR_NULL;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k8_pool) || !aligned16(v8_pool) ||
      !aligned16(k_scale) || !aligned16(v_scale))
    return ATTN_ERR_ALIGN;
  return hip_status(lcat::launch_kv_quantize_fp8(k_pool, v_pool, k8_pool, v8_pool, k_scale,
                                                 v_scale, n_blocks,
                                                 static_cast<hipStream_t>(stream)));
}

int rope_apply(void *x, const int32_t *positions, int S, int H, int D, float base, void *stream) {
  if (S < 0 || H <= 0 || D <= 0) return ATTN_ERR_SHAPE;
  if (D % 16 || D > 256) return ATTN_ERR_UNSUPPORTED;
  if (!(base > 0.f)) return ATTN_ERR_SHAPE;
  if (S == 0) return ATTN_OK;
  if (!x || !positions) return ATTN_ERR_NULL;
  if (!aligned16(x)) return ATTN_ERR_ALIGN;
  return hip_status(lcat::launch_rope(x, H, nullptr, 0, positions, S, D, base,
                                      static_cast<hipStream_t>(stream)));
}

int rope_apply_qk(void *q, void *k, const int32_t *positions, int S, int Hq, int Hkv, int D,
                  float base, void *stream) {
  if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return ATTN_ERR_SHAPE;
  if (D % 16 || D > 256) return ATTN_ERR_UNSUPPORTED;
  if (!(base > 0.f)) return ATTN_ERR_SHAPE;
  if (S == 0) return ATTN_OK;
  if (!q || !k || !positions) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k)) return ATTN_ERR_ALIGN;
  const long long nq = (long long)S * Hq * D * 2, nk = (long long)S * Hkv * D * 2;
  const char *a = static_cast<const char *>(q), *c = static_cast<const char *>(k);
  if (a < c + nk && c < a + nq) return ATTN_ERR_SHAPE;   // q and k overlap
  return hip_status(lcat::launch_rope(q, Hq, k, Hkv, positions, S, D, base,
                                      static_cast<hipStream_t>(stream)));
}

int seq_to_head_permute(const void *in, void *out, int SP, int S_loc, int H_tot, int D, int rank,
                        int elem_bytes, void *stream) {
  if (SP <= 0 || S_loc < 0 || H_tot <= 0 || D <= 0 || H_tot % SP) return ATTN_ERR_SHAPE;
  if (rank < 0 || rank >= SP) return ATTN_ERR_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
    return ATTN_ERR_DTYPE;
  if (S_loc == 0) return ATTN_OK;
  if (!in || !out) return ATTN_ERR_NULL;
  const char *a = static_cast<const char *>(in);
  char *c = static_cast<char *>(out);
  const long long out_bytes = (long long)SP * S_loc * (H_tot / SP) * D * elem_bytes;
  const long long in_bytes = (long long)SP * S_loc * H_tot * D * elem_bytes;
  if (!(c + out_bytes <= a || a + in_bytes <= c)) return ATTN_ERR_SHAPE;   // overlap
  return hip_status(lcat::launch_permute(in, out, SP, S_loc, H_tot, D, rank, elem_bytes,
                                         static_cast<hipStream_t>(stream)));
}

int head_to_seq_permute(const void *in, void *out, int SP, int S_loc, int H_tot, int D, int rank,
                        int elem_bytes, void *stream) {
  if (SP <= 0 || S_loc < 0 || H_tot <= 0 || D <= 0 || H_tot % SP) return ATTN_ERR_SHAPE;
  if (rank < 0 || rank >= SP) return ATTN_ERR_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
    return ATTN_ERR_DTYPE;
  if (S_loc == 0) return ATTN_OK;
  if (!in || !out) return ATTN_ERR_NULL;
  const char *a = static_cast<const char *>(in);
  char *c = static_cast<char *>(out);
  const long long in_bytes = (long long)SP * S_loc * (H_tot / SP) * D * elem_bytes;
  const long long out_bytes = (long long)SP * S_loc * H_tot * D * elem_bytes;
  if (!(c + out_bytes <= a || a + in_bytes <= c)) return ATTN_ERR_SHAPE;   // overlap
  return hip_status(lcat::launch_unpermute(in, out, SP, S_loc, H_tot, D, rank, elem_bytes,
                                           static_cast<hipStream_t>(stream)));
}

int seq_to_head_permute_qkv(const void *q_in, const void *k_in, const void *v_in, void *q_out,
                            void *k_out, void *v_out, int SP, int S_loc, int Hq_tot, int Hkv_tot,
                            int D, int rank, int elem_bytes, void *stream) {
  if (SP <= 0 || S_loc < 0 || Hq_tot <= 0 || Hkv_tot <= 0 || D <= 0 || Hq_tot % SP ||
      Hkv_tot % SP)
    return ATTN_ERR_SHAPE;
  if (rank < 0 || rank >= SP) return ATTN_ERR_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
    return ATTN_ERR_DTYPE;
  if (S_loc == 0) return ATTN_OK;
  const void *in[3] = {q_in, k_in, v_in};
  void *out[3] = {q_out, k_out, v_out};
  const int H[3] = {Hq_tot, Hkv_tot, Hkv_tot};
  for (int t = 0; t < 3; ++t)
    if (!in[t] || !out[t]) return ATTN_ERR_NULL;
  if (!qkv_disjoint(in, out, H, SP, S_loc, D, elem_bytes)) return ATTN_ERR_SHAPE;
  return hip_status(lcat::launch_permute_qkv(in, out, H, SP, S_loc, D, rank, elem_bytes,
                                             static_cast<hipStream_t>(stream)));
}

int seq_to_head_permute_qkv_rope(const void *q_in, const void *k_in, const void *v_in,
                                 void *q_out, void *k_out, void *v_out, const int32_t *positions,
                                 int SP, int S_loc, int Hq_tot, int Hkv_tot, int D, int rank,
                                 float base, void *stream) {
  if (SP <= 0 || S_loc < 0 || Hq_tot <= 0 || Hkv_tot <= 0 || D <= 0 || Hq_tot % SP ||
      Hkv_tot % SP)
    return ATTN_ERR_SHAPE;
  if (rank < 0 || rank >= SP) return ATTN_ERR_SHAPE;
  if (D % 16 || D > 256) return ATTN_ERR_UNSUPPORTED;
  if (!(base > 0.f)) return ATTN_ERR_SHAPE;
  if (S_loc == 0) return ATTN_OK;
  const void *in[3] = {q_in, k_in, v_in};
  void *out[3] = {q_out, k_out, v_out};
  const int H[3] = {Hq_tot, Hkv_tot, Hkv_tot};
  if (!positions) return ATTN_ERR_NULL;
  for (int t = 0; t < 3; ++t) {
    if (!in[t] || !out[t]) return ATTN_ERR_NULL;
    if (!aligned16(in[t]) || !aligned16(out[t])) return ATTN_ERR_ALIGN;
  }
  if (!qkv_disjoint(in, out, H, SP, S_loc, D, 2)) return ATTN_ERR_SHAPE;
  return hip_status(lcat::launch_permute_qkv_rope(in, out, H, positions, SP, S_loc, D, rank, base,
                                                  static_cast<hipStream_t>(stream)));
}

long long cp_shard_tokens(long long S, int N, int rank, int mode) {
  lcat::CpMap m{};
  long long n = 0;
  if (mode != ATTN_CP_CONTIGUOUS && mode != ATTN_CP_STRIPED && mode != ATTN_CP_ZIGZAG)
    return -ATTN_ERR_UNSUPPORTED;
  return cp_map(S, N, rank, mode, m, n) ? n : -ATTN_ERR_SHAPE;
}

static int cp_copy(const void *in, void *out, int32_t *positions, long long S, int H, int D,
                   int elem_bytes, int N, int rank, int mode, int scatter, void *stream) {
  if (S < 0 || H <= 0 || D <= 0) return ATTN_ERR_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
    return ATTN_ERR_DTYPE;
  if (mode != ATTN_CP_CONTIGUOUS && mode != ATTN_CP_STRIPED && mode != ATTN_CP_ZIGZAG)
    return ATTN_ERR_UNSUPPORTED;
  lcat::CpMap m{};
  long long n_tok = 0;
  if (!cp_map(S, N, rank, mode, m, n_tok)) return ATTN_ERR_SHAPE;
  if (S == 0) return ATTN_OK;
  if (!in || !out) return ATTN_ERR_NULL;
  const long long row = (long long)H * D * elem_bytes;
  const char *a = static_cast<const char *>(in);
  const char *c = static_cast<const char *>(out);
  const long long in_bytes = (scatter ? n_tok : S) * row, out_bytes = (scatter ? S : n_tok) * row;
  if (!(c + out_bytes <= a || a + in_bytes <= c)) return ATTN_ERR_SHAPE;   // overlap
  return hip_status(lcat::launch_cp_copy(in, out, m, n_tok, row, scatter, positions,
                                         static_cast<hipStream_t>(stream)));
}

int cp_shard(const void *full, void *shard, int32_t *positions, long long S, int H, int D,
             int elem_bytes, int N, int rank, int mode, void *stream) {
  return cp_copy(full, shard, positions, S, H, D, elem_bytes, N, rank, mode, 0, stream);
}

int cp_unshard(const void *shard, void *full, long long S, int H, int D, int elem_bytes, int N,
               int rank, int mode, void *stream) {
  return cp_copy(shard, full, nullptr, S, H, D, elem_bytes, N, rank, mode, 1, stream);
}

int attn_key_limits(const int32_t *q_pos, const int32_t *k_pos, int32_t *key_limit, int B, int Sq,
                    int Sk, void *stream) {
  if (B < 0 || Sq < 0 || Sk < 0) return ATTN_ERR_SHAPE;
  if (B == 0 || Sq == 0) return ATTN_OK;
  if (!q_pos || !key_limit || (Sk > 0 && !k_pos)) return ATTN_ERR_NULL;
  return hip_status(lcat::launch_key_limits(q_pos, k_pos, key_limit, B, Sq, Sk,
                                            static_cast<hipStream_t>(stream)));
}

int attn_prefill_limited(const void *q, const void *k, const void *v, const int32_t *key_limit,
                         void *o, float *lse, int B, int Sq, int Sk, int Hq, int Hkv, int D,
                         float scale, int accumulate, void *stream) {
  if (B < 0 || Sq < 0 || Sk <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return ATTN_ERR_SHAPE;
  if (D != kHeadDim || !group_ok(Hq, Hkv)) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || Sq == 0) return ATTN_OK;
  if (!q || !k || !v || !o || !key_limit || (accumulate && !lse)) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_ALIGN;
  lcat::PrefillParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.Sq = Sq; p.Sk = Sk; p.Hq = Hq; p.Hkv = Hkv;
  p.causal = 1;
  p.key_limit = key_limit;
  p.accumulate = accumulate != 0;
  p.scale = scale;
  return hip_status(lcat::launch_prefill_bf16(p, false, static_cast<hipStream_t>(stream)));
}

int attn_merge(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b, void *o,
               float *lse, int B, int S, int H, int D, void *stream) {
  if (B < 0 || S < 0 || H <= 0 || D <= 0) return ATTN_ERR_SHAPE;
  if (D % 8 || 64 % (D / 8)) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || S == 0) return ATTN_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o) return ATTN_ERR_NULL;
  if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o)) return ATTN_ERR_ALIGN;
  // o may be o_a or o_b exactly (in place), but no other overlap
  const long long ob_ = (long long)B * S * H * D * 2, lb_ = (long long)B * S * H * 4;
  auto part = [](const void *x, long long nx, const void *y, long long ny) {
    const char *a = static_cast<const char *>(x), *b = static_cast<const char *>(y);
    return a != b && !(a + nx <= b || b + ny <= a);
  };
  if (part(o, ob_, o_a, ob_) || part(o, ob_, o_b, ob_)) return ATTN_ERR_SHAPE;
  if (lse && (part(lse, lb_, lse_a, lb_) || part(lse, lb_, lse_b, lb_))) return ATTN_ERR_SHAPE;
  return hip_status(lcat::launch_merge(o_a, lse_a, o_b, lse_b, o, lse, B, S, H, D,
                                       static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// Internal launch interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lcat {

// Causal / non-causal tiled attention with bf16 MFMA, head_dim 128.
// Dense mode: K/V are [B][Sk][Hkv][128].  Paged mode: K/V come from the
// block pool through block_table, query row i sits at position
// ctx_before[b] + i and the key count is ctx_before[b] + Sq.
struct PrefillParams {
  const void *q;            // [B][Sq][Hq][128] bf16
  const void *k;            // dense K or k_pool
  const void *v;            // dense V or v_pool
  void *o;                  // [B][Sq][Hq][128] bf16
  float *lse;               // [B][Hq][Sq] or null
  const int32_t *block_table;
  const int32_t *block_head;
  const int32_t *ctx_before;
  int32_t *dev_status;
  int B, Sq, Sk, Hq, Hkv;
  int max_blocks, n_blocks, kv_head_base;
  int causal;
  float scale;
  const int32_t *key_limit;  // dense only, or null: row i sees keys [0, key_limit[b][i])
  int accumulate;            // with key_limit: merge into the partial already in o / lse
};

hipError_t launch_prefill_bf16(const PrefillParams &p, bool paged, hipStream_t stream);

// Signs of the incoherent-processing rotation x -> (s * x) H of 128-element
// rows (hadamard.h): bit i of neg is set when s_i = -1; on = 0 means no
// rotation.
struct HadamardSigns {
  uint32_t neg[4];
  int on;
};

// Dense prefill with FP8 (e4m3) scores: q and v bf16, k as e4m3 codes with
// one E8M0 scale per 32 head dims (attn_quantize_fp8_blocks), head_dim 128.
// With rot.on, each query row is rotated before it is quantised, and k8 must
// hold the rows of K rotated with the same signs.
struct PrefillFp8Params {
  const void *q;            // [B][S][Hq][128] bf16
  const void *k8;           // [B][S][Hkv][128] e4m3
  const uint8_t *k_scale;   // [B][S][Hkv][4] E8M0
  const void *v;            // [B][S][Hkv][128] bf16
  void *o;                  // [B][S][Hq][128] bf16
  float *lse;               // [B][Hq][S] or null
  int B, S, Hq, Hkv;
  int causal;
  float scale;
  HadamardSigns rot;
};

hipError_t launch_prefill_fp8(const PrefillFp8Params &p, hipStream_t stream);

// Dense prefill with both products on FP8: q bf16, k as above, v as e4m3
// codes in the dimension-major layout of attn_quantize_fp8_v (S64 = S rounded
// up to 64 keys) with one E8M0 scale per (dim, 32 keys), head_dim 128.
struct PrefillFp8PvParams {
  const void *q;            // [B][S][Hq][128] bf16
  const void *k8;           // [B][S][Hkv][128] e4m3
  const uint8_t *k_scale;   // [B][S][Hkv][4] E8M0
  const void *v8t;          // [B][Hkv][128][S64] e4m3
  const uint8_t *v_scale;   // [B][Hkv][S64 / 64][256] E8M0 (tile layout)
  void *o;                  // [B][S][Hq][128] bf16
  float *lse;               // [B][Hq][S] or null
  int B, S, Hq, Hkv;
  int causal;
  float scale;
  HadamardSigns rot;
};

hipError_t launch_prefill_fp8_pv(const PrefillFp8PvParams &p, hipStream_t stream);

// V [B][S][Hkv][128] bf16 -> v8t and v_scale as PrefillFp8PvParams reads them.
hipError_t launch_quantize_fp8_v(const void *v, void *v8t, uint8_t *v_scale, int B, int S, int Hkv,
                                 hipStream_t stream);

// Block quantisation: x [n_blocks * 32] bf16 -> e4m3 codes (same count) and
// one E8M0 scale byte per block of 32 consecutive values.
hipError_t launch_quantize_fp8_blocks(const void *x, void *codes, uint8_t *scales,
                                      long long n_blocks, hipStream_t stream);

// Rows of 128 bf16 values rotated by (s * x) H (hadamard.h), then block
// quantised as above: codes [n_rows][128], scales [n_rows][4].
hipError_t launch_quantize_fp8_rotated(const void *x, void *codes, uint8_t *scales,
                                       long long n_rows, HadamardSigns sg, hipStream_t stream);

hipError_t launch_attn_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                           int B, int S, int Hq, int Hkv, int D, int causal, float scale,
                           hipStream_t stream);

hipError_t launch_kv_append(const void *k_new, const void *v_new, void *k_pool, void *v_pool,
                            int n_blocks, const int32_t *block_head, const int32_t *block_table,
                            int max_blocks, const int32_t *start_pos, int T, int B, int Hkv,
                            int kv_head_base, int32_t *dev_status, hipStream_t stream);

struct DecodeParams {
  const void *q;            // [B][Hq][128]
  const void *k_pool;       // [n_blocks][64][128] (bf16, or e4m3 bytes when fp8)
  const void *v_pool;       // [n_blocks][128][64]
  const float *k_scale;     // fp8: [n_blocks][64] per-token K scales
  const float *v_scale;     // fp8: [n_blocks][64] per-token V scales
  int fp8;
  const int32_t *block_head;
  const int32_t *block_table;
  const int32_t *ctx_len;
  void *o;                  // [B][Hq][128]
  float *lse;               // [B][Hq] or null
  float *ws;                // split records (132 floats each), see launch_decode
  int32_t *dev_status;
  int B, Hq, Hkv, max_blocks, n_blocks, kv_head_base;
  int split_tokens, n_split;   // fixed splits (stream_waves == 0)
  int stream_waves;            // > 0: equal-share split over this many waves
  float scale;
};

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream);

// bf16 pools -> e4m3 pools (k8 [n][64][128], v8 [n][128][64]) with per-token
// scales k_scale / v_scale [n][64].
hipError_t launch_kv_quantize_fp8(const void *k_pool, const void *v_pool, void *k8, void *v8,
                                  float *k_scale, float *v_scale, int n_blocks,
                                  hipStream_t stream);

// attn_kv_append into the fp8 pools, quantising each appended token.
hipError_t launch_kv_append_fp8(const void *k_new, const void *v_new, void *k8, void *v8,
                                float *k_scale, float *v_scale, int n_blocks,
                                const int32_t *block_head, const int32_t *block_table,
                                int max_blocks, const int32_t *start_pos, int T, int B, int Hkv,
                                int kv_head_base, int32_t *dev_status, hipStream_t stream);

// RoPE in place on x [S][H][D] and, when H2 > 0, on x2 [S][H2][D] at the
// same positions (one launch, one (cos, sin) table per token).
hipError_t launch_rope(void *x, int H, void *x2, int H2, const int32_t *positions, int S, int D,
                       float base, hipStream_t stream);

hipError_t launch_permute(const void *in, void *out, int SP, int S_loc, int H_tot, int D, int rank,
                          int elem_bytes, hipStream_t stream);

// The inverse: [SP*S_loc][H_tot/SP][D] -> rank's head slice of [SP][S_loc][H_tot][D].
hipError_t launch_unpermute(const void *in, void *out, int SP, int S_loc, int H_tot, int D,
                            int rank, int elem_bytes, hipStream_t stream);

// Q, K and V (head counts H_tot[0..2]) in one launch.
hipError_t launch_permute_qkv(const void *const in[3], void *const out[3], const int H_tot[3],
                              int SP, int S_loc, int D, int rank, int elem_bytes,
                              hipStream_t stream);

// The same relayout of bf16 Q, K and V with RoPE at positions[t] (t in global
// token order) applied to Q and K on the way; D % 16 == 0, D <= 256, all
// pointers 16-byte aligned.
hipError_t launch_permute_qkv_rope(const void *const in[3], void *const out[3], const int H_tot[3],
                                   const int32_t *positions, int SP, int S_loc, int D, int rank,
                                   float base, hipStream_t stream);

// Context-parallel shard of a sequence: local token i is global token
//   i < len_a ? start_a + i * stride : start_b + (i - len_a) * stride.
struct CpMap {
  long long start_a, len_a, start_b, stride;
};

// Gather (scatter = 0: full [S][row] -> shard [n_tok][row]) or scatter back
// (scatter = 1); positions (nullable) receives the global index of each
// local token.
hipError_t launch_cp_copy(const void *in, void *out, const CpMap &m, long long n_tok,
                          long long row_bytes, int scatter, int32_t *positions,
                          hipStream_t stream);

// lim[b][i] = #{j : k_pos[b][j] <= q_pos[b][i]} for ascending k_pos.
hipError_t launch_key_limits(const int32_t *q_pos, const int32_t *k_pos, int32_t *lim, int B,
                             int Sq, int Sk, hipStream_t stream);

// Merge of two normalised partial attention results (bf16 O, fp32 LSE).
hipError_t launch_merge(const void *oa, const float *la, const void *ob, const float *lb, void *o,
                        float *lse, int B, int S, int H, int D, hipStream_t stream);

}  // namespace lcat

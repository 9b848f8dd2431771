/*
 * CPU oracle for exact long-context attention — TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, the smoke check and the benchmark's CPU-baseline leg may load
 * this library.  The HIP product path never links or calls it, and it shares
 * no code, header, table or constant with that path.
 *
 * Everything is evaluated in fp64 with plain loops, in the order the pages'
 * definitions state, with no blocking, fusion or reordering:
 *
 *  - attention: the naive definition S = Q K^T * scale, A = softmax(S),
 *    out = A V ("Flash Attention and distributed inference", §18.2), one query
 *    row at a time, with the softmax taken in its three-pass form (max, then
 *    denominator, then weighted sum; same chapter, §18.3).  The online
 *    recurrence the GPU uses is never used here.
 *  - rotary embedding at absolute token positions (Ulysses inference article,
 *    §3.2 and §5.3): angle p * base^(-2i/D), rotate-half pairing (i, i+D/2).
 *  - sequence-shard -> head-shard relayout (same article, §2.2), and its
 *    inverse for the attention output (head shard back to sequence shards).
 *  - gather of a head-sharded paged KV cache (same article, §2.3) into
 *    contiguous order.
 *  - attention with the causal mask on token positions, for the sequence
 *    shards of context-parallel ranks ("LLM推理中的多卡切分", §3.5).
 *
 * Inputs may be fp64, fp32 or bf16 bit patterns; they are widened to fp64
 * exactly on read.  OpenMP splits independent (batch, row, head) items only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2 };

static double widen(const void *base, int dtype, int64_t idx) {
  if (dtype == ORC_F64) return ((const double *)base)[idx];
  if (dtype == ORC_F32) return (double)((const float *)base)[idx];
  uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/*
 * Attention for selected query rows.
 *   q_rows : [B][R][Hq][D]   the query vectors of the R selected rows
 *   k, v   : [B][Sk][Hkv][D] keys and values (each with its own dtype code)
 *   key_limit : [B][R]       row r of batch b may attend keys 0 .. key_limit-1
 *                            (this single rule expresses non-causal, causal,
 *                            chunked and decode masks; the caller computes it)
 *   out    : [B][R][Hq][D]   fp64
 *   lse    : [B][Hq][R]      natural-log log-sum-exp of the scaled scores
 * Query head h reads KV head h / (Hq/Hkv) (grouped-query attention).
 * A row with no allowed key gets out = NaN and lse = -inf.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_attention_rows(const void *q_rows, int q_dtype, const void *k, int k_dtype,
                          const void *v, int v_dtype, int64_t B, int64_t R, int64_t Sk, int64_t Hq,
                          int64_t Hkv, int64_t D, const int64_t *key_limit, double scale,
                          double *out, double *lse) {
  if (!q_rows || !k || !v || !key_limit || !out || !lse) return -1;
  if (B < 0 || R < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return -1;
  const int64_t group = Hq / Hkv;
  const int64_t n_items = B * R * Hq;
  int failed = 0;
#pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
    if (!s) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t item = 0; item < n_items; ++item) {
      if (!s) continue;
      const int64_t h = item % Hq;
      const int64_t r = (item / Hq) % R;
      const int64_t b = item / (Hq * R);
      const int64_t g = h / group;
      int64_t lim = key_limit[b * R + r];
      if (lim > Sk) lim = Sk;
      double *o = out + ((b * R + r) * Hq + h) * D;
      const int64_t q_off = ((b * R + r) * Hq + h) * D;
      if (lim <= 0) {
        for (int64_t d = 0; d < D; ++d) o[d] = NAN;
        lse[(b * Hq + h) * R + r] = -INFINITY;
        continue;
      }
      /* scores of this row: s_j = scale * <q_i, k_j> */
      for (int64_t j = 0; j < lim; ++j) {
        const int64_t k_off = ((b * Sk + j) * Hkv + g) * D;
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d) acc += widen(q_rows, q_dtype, q_off + d) * widen(k, k_dtype, k_off + d);
        s[j] = scale * acc;
      }
      /* pass 1: maximum */
      double m = -INFINITY;
      for (int64_t j = 0; j < lim; ++j)
        if (s[j] > m) m = s[j];
      /* pass 2: denominator */
      double z = 0.0;
      for (int64_t j = 0; j < lim; ++j) z += exp(s[j] - m);
      /* pass 3: normalised weights times values */
      for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
      for (int64_t j = 0; j < lim; ++j) {
        const double a = exp(s[j] - m) / z;
        const int64_t v_off = ((b * Sk + j) * Hkv + g) * D;
        for (int64_t d = 0; d < D; ++d) o[d] += a * widen(v, v_dtype, v_off + d);
      }
      lse[(b * Hq + h) * R + r] = m + log(z);
    }
    free(s);
  }
  return failed ? -1 : 0;
}

/*
 * Attention with the causal mask stated on token positions, for query and
 * key sets that are arbitrary subsets of one sequence (the shards that
 * context-parallel ranks hold: contiguous, striped or zigzag; "LLM推理中的
 * 多卡切分", §3.5).  A query at position P may attend exactly the keys whose
 * position is <= P, wherever those keys sit in the key array.
 *   q      : [B][Sq][Hq][D],  q_pos : [B][Sq]
 *   k, v   : [B][Sk][Hkv][D], k_pos : [B][Sk]
 *   out    : [B][Sq][Hq][D] fp64, lse : [B][Hq][Sq]
 * Rows with no allowed key get out = NaN and lse = -inf.  Three-pass softmax
 * as in oracle_attention_rows.
 */
int oracle_attention_positions(const void *q, int q_dtype, const void *k, int k_dtype,
                               const void *v, int v_dtype, int64_t B, int64_t Sq, int64_t Sk,
                               int64_t Hq, int64_t Hkv, int64_t D, const int64_t *q_pos,
                               const int64_t *k_pos, double scale, double *out, double *lse) {
  if (!q || !k || !v || !q_pos || !k_pos || !out || !lse) return -1;
  if (B < 0 || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return -1;
  const int64_t group = Hq / Hkv;
  const int64_t n_items = B * Sq * Hq;
  int failed = 0;
#pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
    int64_t *key = (int64_t *)malloc(sizeof(int64_t) * (size_t)(Sk > 0 ? Sk : 1));
    if (!s || !key) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t item = 0; item < n_items; ++item) {
      if (!s || !key) continue;
      const int64_t h = item % Hq;
      const int64_t r = (item / Hq) % Sq;
      const int64_t b = item / (Hq * Sq);
      const int64_t g = h / group;
      double *o = out + ((b * Sq + r) * Hq + h) * D;
      const int64_t q_off = ((b * Sq + r) * Hq + h) * D;
      /* the allowed keys: position not after the query's */
      int64_t n = 0;
      for (int64_t j = 0; j < Sk; ++j)
        if (k_pos[b * Sk + j] <= q_pos[b * Sq + r]) key[n++] = j;
      if (n == 0) {
        for (int64_t d = 0; d < D; ++d) o[d] = NAN;
        lse[(b * Hq + h) * Sq + r] = -INFINITY;
        continue;
      }
      for (int64_t t = 0; t < n; ++t) {
        const int64_t k_off = ((b * Sk + key[t]) * Hkv + g) * D;
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d) acc += widen(q, q_dtype, q_off + d) * widen(k, k_dtype, k_off + d);
        s[t] = scale * acc;
      }
      double m = -INFINITY;
      for (int64_t t = 0; t < n; ++t)
        if (s[t] > m) m = s[t];
      double z = 0.0;
      for (int64_t t = 0; t < n; ++t) z += exp(s[t] - m);
      for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
      for (int64_t t = 0; t < n; ++t) {
        const double a = exp(s[t] - m) / z;
        const int64_t v_off = ((b * Sk + key[t]) * Hkv + g) * D;
        for (int64_t d = 0; d < D; ++d) o[d] += a * widen(v, v_dtype, v_off + d);
      }
      lse[(b * Hq + h) * Sq + r] = m + log(z);
    }
    free(s);
    free(key);
  }
  return failed ? -1 : 0;
}

/*
 * Rotary embedding at absolute positions, fp64 throughout.
 *   x   : [S][H][D] (any supported dtype), pos : [S] absolute positions
 *   out : [S][H][D] fp64
 * For i < D/2, theta_i = base^(-2i/D), a = pos[t] * theta_i:
 *   out[i]       = x[i] cos a - x[i+D/2] sin a
 *   out[i+D/2]   = x[i+D/2] cos a + x[i] sin a
 */
int oracle_rope(const void *x, int dtype, const int64_t *pos, int64_t S, int64_t H, int64_t D,
                double base, double *out) {
  if (!x || !pos || !out || S < 0 || H <= 0 || D <= 0 || (D & 1)) return -1;
  const int64_t half = D / 2;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < S; ++t) {
    for (int64_t h = 0; h < H; ++h) {
      const int64_t off = (t * H + h) * D;
      for (int64_t i = 0; i < half; ++i) {
        const double theta = pow(base, -2.0 * (double)i / (double)D);
        const double a = (double)pos[t] * theta;
        const double c = cos(a), sn = sin(a);
        const double x0 = widen(x, dtype, off + i);
        const double x1 = widen(x, dtype, off + i + half);
        out[off + i] = x0 * c - x1 * sn;
        out[off + i + half] = x1 * c + x0 * sn;
      }
    }
  }
  return 0;
}

/*
 * Sequence-shard -> head-shard relayout for one rank.
 *   in  : [SP][S_loc][H_tot][D] elements of elem_bytes bytes
 *   out : [SP*S_loc][H_tot/SP][D]
 *   out[k*S_loc + s][h][:] = in[k][s][rank*(H_tot/SP) + h][:]
 * Payload bytes are copied unchanged.
 */
int oracle_permute(const void *in, void *out, int64_t SP, int64_t S_loc, int64_t H_tot,
                   int64_t D, int64_t rank, int64_t elem_bytes) {
  if (!in || !out || SP <= 0 || S_loc < 0 || H_tot <= 0 || D <= 0 || elem_bytes <= 0) return -1;
  if (H_tot % SP || rank < 0 || rank >= SP) return -1;
  const int64_t H_loc = H_tot / SP;
  const int64_t row = D * elem_bytes;
  const char *src = (const char *)in;
  char *dst = (char *)out;
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < SP; ++k)
    for (int64_t s = 0; s < S_loc; ++s)
      for (int64_t h = 0; h < H_loc; ++h) {
        const int64_t src_idx = (k * S_loc + s) * H_tot + rank * H_loc + h;
        const int64_t dst_idx = (k * S_loc + s) * H_loc + h;
        memcpy(dst + dst_idx * row, src + src_idx * row, (size_t)row);
      }
  return 0;
}

/*
 * Head-shard -> sequence-shard relayout for one rank: the second exchange of
 * the Ulysses inference article (§2.2), which returns the attention output of
 * this rank's heads to the sequence shards; §2.3 places each head by its
 * global index.
 *   in  : [SP*S_loc][H_tot/SP][D]   this rank's heads, global token order
 *   out : [SP][S_loc][H_tot][D]     the SP sequence shards, all heads
 *   out[k][s][rank*(H_tot/SP) + h][:] = in[k*S_loc + s][h][:]
 * Only this rank's head slice of out is written; every other byte of out is
 * left as it was.  Payload bytes are copied unchanged.
 */
int oracle_unpermute(const void *in, void *out, int64_t SP, int64_t S_loc, int64_t H_tot,
                     int64_t D, int64_t rank, int64_t elem_bytes) {
  if (!in || !out || SP <= 0 || S_loc < 0 || H_tot <= 0 || D <= 0 || elem_bytes <= 0) return -1;
  if (H_tot % SP || rank < 0 || rank >= SP) return -1;
  const int64_t H_loc = H_tot / SP;
  const int64_t row = D * elem_bytes;
  const char *src = (const char *)in;
  char *dst = (char *)out;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < SP * S_loc; ++t) {
    const int64_t k = t / S_loc, s = t % S_loc;
    for (int64_t h = 0; h < H_loc; ++h) {
      const int64_t src_idx = t * H_loc + h;
      const int64_t dst_idx = (k * S_loc + s) * H_tot + rank * H_loc + h;
      memcpy(dst + dst_idx * row, src + src_idx * row, (size_t)row);
    }
  }
  return 0;
}

/*
 * Gather a paged, head-sharded KV cache into contiguous order (bit copies).
 *   k_pool : [n_blocks][64][D] bf16 bits   (token-major blocks)
 *   v_pool : [n_blocks][D][64] bf16 bits   (dimension-major blocks)
 *   table  : [B][Hkv][max_blocks]           logical block -> physical block
 *   n_tok  : [B]                            tokens to gather per request
 *   k_out, v_out : [B][T_max][Hkv][D]       token t of request b, head g:
 *      k_out[b][t][g][d] = k_pool[table[b][g][t/64]][t%64][d]
 *      v_out[b][t][g][d] = v_pool[table[b][g][t/64]][d][t%64]
 * Returns -2 if a table entry needed for a gathered token is out of range.
 */
int oracle_paged_gather(const uint16_t *k_pool, const uint16_t *v_pool, int64_t n_blocks,
                        const int32_t *table, int64_t B, int64_t Hkv, int64_t max_blocks,
                        const int64_t *n_tok, int64_t T_max, int64_t D, uint16_t *k_out,
                        uint16_t *v_out) {
  if (!k_pool || !v_pool || !table || !n_tok || !k_out || !v_out) return -1;
  const int64_t BT = 64;
  int bad = 0;
  for (int64_t b = 0; b < B; ++b) {
    if (n_tok[b] > T_max || n_tok[b] > max_blocks * BT) return -1;
    for (int64_t t = 0; t < n_tok[b]; ++t)
      for (int64_t g = 0; g < Hkv; ++g) {
        const int64_t blk = table[(b * Hkv + g) * max_blocks + t / BT];
        if (blk < 0 || blk >= n_blocks) {
          bad = 1;
          continue;
        }
        const int64_t slot = t % BT;
        for (int64_t d = 0; d < D; ++d) {
          k_out[((b * T_max + t) * Hkv + g) * D + d] = k_pool[(blk * BT + slot) * D + d];
          v_out[((b * T_max + t) * Hkv + g) * D + d] = v_pool[(blk * D + d) * BT + slot];
        }
      }
  }
  return bad ? -2 : 0;
}

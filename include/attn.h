/*
 * libattn — exact long-context attention for AMD MI355X (gfx950), C ABI.
 *
 * Sources for what each call computes (pages cited by title and section):
 *  [FA18]    "Flash Attention and distributed inference: memory hierarchy and
 *            multi-GPU" (Transformer anatomy, chapter 18): §18.2 naive
 *            attention, §18.3 tiling with the online softmax (running max m,
 *            denominator l, rescaled output accumulator), §18.4 deferred
 *            normalisation and the Q-outer loop order.
 *  [ULY]     Ulysses sequence parallelism moved into long-context inference
 *            (kwkr.cn article): §2.2 sequence-shard -> head-shard relayout,
 *            §2.3 head-sharded KV cache in per-head blocks tagged with a
 *            global head index, §3.2 RoPE at absolute token positions,
 *            §3.5 1e-3 numeric alignment, §5.3 full-sequence causal mask.
 *  [MGP]     "LLM推理中的多卡切分" (multi-GPU partitioning in LLM inference):
 *            §2.1 request-token -> KV-slot allocation, §2.2 chunked prefill,
 *            §3.5 / §3.5.1 context parallelism (ring, striped, zigzag).
 *
 * Conventions shared by every call
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates or frees device memory and keeps no mutable state, so
 *    calls are thread-safe.  (attn_decode_noalloc is the one exception: it
 *    uses a fixed device array of the library, see there.)  `stream` is a hipStream_t passed as void*
 *    (NULL = the default stream).  Every call only enqueues work on `stream`
 *    and returns without synchronising.  Grid sizes come from host arguments
 *    only; device arrays (ctx_before, ctx_len, tables) are read on the device.
 *  - Return value: ATTN_OK (0) or a synchronous error code below.  Argument
 *    errors are detected before anything is enqueued.  A failed launch is
 *    reported as ATTN_ERR_HIP.
 *  - Device-detected errors (a block tag that is not the expected global KV
 *    head, a block id outside [0, n_blocks)) store a non-zero ATTN_DEV_* code
 *    into *dev_status (if dev_status is not NULL); the caller reads it after
 *    synchronising.  Output rows touched by such a block are undefined.
 *  - bf16 is IEEE bfloat16 (1-8-7); fp32 is IEEE binary32.  Head dimension D
 *    is 128 for every bf16 path.  Tensors are dense, row-major, innermost
 *    index last, with 16-byte aligned base pointers.
 *  - Paged KV cache (per [ULY] §2.3): a pool of n_blocks blocks of 64 tokens,
 *    each block holding ONE KV head:
 *        k_pool [n_blocks][64][D]   token-major  (row = one token)
 *        v_pool [n_blocks][D][64]   dimension-major (row = one channel)
 *        block_head  [n_blocks]           int32 global KV-head tag per block
 *        block_table [B][Hkv][max_blocks] int32 physical block of logical
 *                    block j (tokens 64j..64j+63) of request b, local KV head g
 *    Local KV head g of this GPU is global head kv_head_base + g; every block
 *    read or written for (b, g) must carry that tag.
 */
#ifndef LCAT_ATTN_H
#define LCAT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* negative size, Hq % Hkv != 0, H_tot % SP != 0, rank out of range */
  ATTN_ERR_DTYPE = 3,       /* unknown dtype / element size */
  ATTN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  ATTN_ERR_UNSUPPORTED = 5, /* valid but not implemented (e.g. D != 128 on a bf16 path) */
  ATTN_ERR_WORKSPACE = 6,   /* decode workspace missing or too small */
  ATTN_ERR_HIP = 7,         /* the HIP runtime rejected a launch */
  ATTN_ERR_SCRATCH = 8      /* attn_decode_noalloc: more than ATTN_NOALLOC_SCRATCH_BYTES needed */
};

enum attn_dtype { ATTN_DTYPE_F32 = 0, ATTN_DTYPE_BF16 = 1 };

enum attn_dev_status { ATTN_DEV_OK = 0, ATTN_DEV_BAD_TAG = 1, ATTN_DEV_BAD_BLOCK = 2 };

/* Context-parallel splits of a sequence over N ranks ([MGP] §3.5, §3.5.1). */
enum attn_cp_mode {
  ATTN_CP_CONTIGUOUS = 0, /* ring attention: N consecutive blocks */
  ATTN_CP_STRIPED = 1,    /* round-robin: tokens with index mod N == rank; S % N == 0 */
  ATTN_CP_ZIGZAG = 2      /* in-seq-split: 2N blocks, rank i holds blocks i and 2N-1-i; S >= 2N */
};

/*
 * attn_prefill — exact softmax attention over dense Q/K/V ([FA18] §18.2 for
 * the result, §18.3-§18.4 for the tiled online-softmax evaluation).
 *   q   [B][S][Hq][D]      o [B][S][Hq][D] (same dtype as q)
 *   k,v [B][S][Hkv][D]     lse [B][Hq][S] fp32, natural log, or NULL
 * out[b,i,h,:] = sum_j softmax_j(scale * q_i . k_j) v_j over keys j of KV
 * head h / (Hq/Hkv); with causal != 0 only keys j <= i are visible (global
 * token indices, [ULY] §5.3).  lse[b,h,i] = log sum_j exp(scale * q_i . k_j).
 *   dtype ATTN_DTYPE_BF16: D must be 128, Hq/Hkv must divide 8 or be a
 *         multiple of 8; bf16 MFMA products with fp32 accumulation.  Each
 *         query row is multiplied by scale * log2(e) and rounded to bf16
 *         once, so every product term of a score carries one extra relative
 *         rounding of at most 2^-9 (as large as the bf16 rounding of the
 *         inputs); lse then differs from its exact value by at most 2^-9
 *         times the magnitude of the scores that carry the softmax weight.
 *         P is rounded to bf16 before P V.  The same holds for
 *         attn_chunked_prefill and attn_prefill_limited.
 *   dtype ATTN_DTYPE_F32 : D must be 64 or 128; fp32 arithmetic throughout.
 * S = 0 or B = 0 is a no-op.
 */
int attn_prefill(const void *q, const void *k, const void *v, void *o, float *lse, int B, int S,
                 int Hq, int Hkv, int D, int dtype, int causal, float scale, void *stream);

/*
 * attn_kv_append — write T new tokens per request into the paged cache
 * ([ULY] §2.3 layout; slots follow the request-token -> KV-slot map of
 * [MGP] §2.1).  For request b, local KV head g and t in [0, T):
 *   pos  = start_pos[b] + t,  blk = block_table[b][g][pos / 64]
 *   k_pool[blk][pos % 64][:] = k_new[b][t][g][:]
 *   v_pool[blk][:][pos % 64] = v_new[b][t][g][:]
 *   k_new, v_new [B][T][Hkv][D] bf16; start_pos [B] int32 (device).
 * Blocks must already be assigned in block_table and tagged in block_head;
 * a wrong tag or an out-of-range id sets *dev_status and skips that block.
 */
int attn_kv_append(const void *k_new, const void *v_new, void *k_pool, void *v_pool, int n_blocks,
                   const int32_t *block_head, const int32_t *block_table, int max_blocks,
                   const int32_t *start_pos, int T, int B, int Hkv, int D, int kv_head_base,
                   int32_t *dev_status, void *stream);

/*
 * attn_chunked_prefill — one chunk of C new tokens per request attending to
 * all previously cached tokens plus, causally, to the chunk itself ([MGP]
 * §2.2).  First appends the chunk's K/V (exactly attn_kv_append with
 * start_pos = ctx_before, T = C), then, in stream order, for chunk row i
 * (global position ctx_before[b] + i) attends keys at positions
 * 0 .. ctx_before[b] + i read from the paged cache.
 *   q [B][C][Hq][D] bf16, k_new/v_new [B][C][Hkv][D] bf16,
 *   o [B][C][Hq][D] bf16, lse [B][Hq][C] fp32 or NULL,
 *   ctx_before [B] int32 (device): tokens already cached per request.
 * D must be 128.  C = 0 or B = 0 is a no-op.
 */
int attn_chunked_prefill(const void *q, const void *k_new, const void *v_new, void *k_pool,
                         void *v_pool, int n_blocks, const int32_t *block_head,
                         const int32_t *block_table, int max_blocks, const int32_t *ctx_before,
                         int C, void *o, float *lse, int B, int Hq, int Hkv, int D,
                         int kv_head_base, float scale, int32_t *dev_status, void *stream);

/*
 * attn_decode — one new query token per request over its whole cached
 * context, split over key ranges whose partial (max, denominator, output)
 * triples are merged with the log-sum-exp rescale of [FA18] §18.3.
 *   q [B][Hq][D] bf16, o [B][Hq][D] bf16, lse [B][Hq] fp32 or NULL,
 *   ctx_len [B] int32 (device): cached tokens INCLUDING the new one; every
 *   key 0 .. ctx_len-1 is visible.  Slots past ctx_len are never used in
 *   arithmetic (they may hold NaN).
 *   split_tokens: keys per split, a positive multiple of 64, or 0 = automatic
 *   (the blocks of all requests and KV heads are shared out equally among
 *   256 to 768 waves, about four blocks per wave at the least, so long and
 *   short contexts load the GPU evenly).
 *   workspace: caller-owned device scratch of at least
 *   attn_decode_workspace_bytes(B, Hq, D, max_blocks, split_tokens) bytes.
 * D must be 128 and Hq/Hkv at most 16.  ctx_len[b] = 0 gives o = 0 and
 * lse = -inf for that request.
 */
int attn_decode(const void *q, const void *k_pool, const void *v_pool, int n_blocks,
                const int32_t *block_head, const int32_t *block_table, int max_blocks,
                const int32_t *ctx_len, void *o, float *lse, int B, int Hq, int Hkv, int D,
                int kv_head_base, float scale, int split_tokens, void *workspace,
                size_t workspace_bytes, int32_t *dev_status, void *stream);

/* Workspace bytes attn_decode needs (0 on invalid arguments). */
size_t attn_decode_workspace_bytes(int B, int Hq, int D, int max_blocks, int split_tokens);

/*
 * attn_decode_noalloc — attn_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace, and the same
 * outputs (bit for bit: the same kernels run).  The split records go to a
 * fixed device array of the library, one per GPU, of
 * ATTN_NOALLOC_SCRATCH_BYTES bytes, which each GPU holds from the first call
 * on it until the process ends.  A call whose records need more
 * (attn_decode_workspace_bytes(B, Hq, D, max_blocks, split_tokens) above the
 * maximum; with split_tokens = 0 that is (768 + B) * Hq * 528 bytes) returns
 * ATTN_ERR_SCRATCH and enqueues nothing.  No part of the array needs to start
 * at zero.  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine); the first call on a GPU looks up that GPU's copy of the
 * array, so a caller that captures a graph makes one call on that GPU
 * before capturing (later calls enqueue kernels only).  Every call on one
 * GPU shares its array: calls that overlap on one
 * GPU (on different streams, or from different threads without ordering)
 * race on it and their outputs are undefined; calls ordered on one stream
 * are safe.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (16 << 20)
int attn_decode_noalloc(const void *q, const void *k_pool, const void *v_pool, int n_blocks,
                        const int32_t *block_head, const int32_t *block_table, int max_blocks,
                        const int32_t *ctx_len, void *o, float *lse, int B, int Hq, int Hkv, int D,
                        int kv_head_base, float scale, int split_tokens, int32_t *dev_status,
                        void *stream);

/*
 * FP8 KV cache ([ULY] §5.4 keeps the cache quantised in groups; FA3's FP8
 * path in [FA18] quantises blocks to 8-bit floats).  Reading taken: OCP e4m3
 * codes with one fp32 scale per token — per K row and per V column of each
 * 64-token block — scale = amax / 448, code = x / scale rounded to nearest
 * e4m3 (ties to even, magnitudes clamped to 448), all-zero groups get scale
 * 0 and codes 0.  Dequantised value = e4m3(code) * scale.
 *   k8_pool [n_blocks][64][D] and v8_pool [n_blocks][D][64] bytes (the bf16
 *   layouts with 1-byte elements), k_scale / v_scale [n_blocks][64] fp32.
 *
 * attn_kv_quantize_fp8 — quantise whole bf16 pools into that form.  D = 128.
 *   Codes are fixed by the definition above (IEEE fp32 divisions).
 */
int attn_kv_quantize_fp8(const void *k_pool, const void *v_pool, void *k8_pool, void *v8_pool,
                         float *k_scale, float *v_scale, int n_blocks, int D, void *stream);

/*
 * attn_kv_append_fp8 — attn_kv_append into the FP8 pools: the same token ->
 * slot map, block checks and dev_status codes; each appended token's K row
 * and V vector are quantised with their own scales exactly as
 * attn_kv_quantize_fp8 would ([ULY] §5.4 grouped quantised cache), and no
 * other token's codes or scales change.  k_new, v_new [B][T][Hkv][D] bf16.
 */
int attn_kv_append_fp8(const void *k_new, const void *v_new, void *k8_pool, void *v8_pool,
                       float *k_scale, float *v_scale, int n_blocks, const int32_t *block_head,
                       const int32_t *block_table, int max_blocks, const int32_t *start_pos, int T,
                       int B, int Hkv, int D, int kv_head_base, int32_t *dev_status,
                       void *stream);

/*
 * attn_decode_fp8 — attn_decode over the FP8 cache: the same arguments,
 * splits, workspace (attn_decode_workspace_bytes), tag and block checks and
 * outputs, with the e4m3 pools and their per-token scales in place of the
 * bf16 pools.  Scores use the dequantised keys, P V the dequantised values;
 * q stays bf16.  Reads 16.5 KiB per block and KV head instead of 32 KiB.
 */
int attn_decode_fp8(const void *q, const void *k8_pool, const void *v8_pool, const float *k_scale,
                    const float *v_scale, int n_blocks, const int32_t *block_head,
                    const int32_t *block_table, int max_blocks, const int32_t *ctx_len, void *o,
                    float *lse, int B, int Hq, int Hkv, int D, int kv_head_base, float scale,
                    int split_tokens, void *workspace, size_t workspace_bytes,
                    int32_t *dev_status, void *stream);

/*
 * FP8 scores for prefill ([FA18] §18.5: FA3's FP8 path runs the attention
 * matmuls on 8-bit operands with block quantisation).  Reading taken (the
 * pages fix no format or rule): OCP e4m3 codes, one power-of-two scale per
 * block of 32 consecutive head dims of one token, 2^e with e the smallest
 * integer such that max|x| <= 448 * 2^e (floored at -127), codes = x / 2^e
 * rounded to the nearest e4m3 value, ties to even; the scale is stored as the
 * E8M0 byte e + 127.  attn_prefill_fp8 runs S = Q K^T on FP8 (P V in bf16);
 * attn_prefill_fp8_pv runs both products on FP8.
 *
 * Incoherent processing (the other half of FA3's FP8 path in [FA18] §18.5):
 * `signs`, when not NULL, is a HOST array of 128 values, each +1 or -1
 * (ATTN_ERR_SHAPE otherwise), that the caller draws once.  Q and K rows are
 * then rotated before they are quantised: x -> (s * x) H, H the 128 x 128
 * Sylvester-Hadamard matrix (H[i][j] = (-1)^popcount(i & j)), computed in
 * fp32 as butterflies of span 1, 2, 4, ..., 64 (pairs (i, i + span) with bit
 * `span` of i clear become (a + b, a - b)), so the codes are reproducible.
 * Since H H^T = 128 I the scores keep their values: the query multiplier
 * becomes scale * log2(e) / 128.  K must be quantised with the same signs
 * that the prefill receives; V is not rotated.
 *
 * attn_quantize_fp8_blocks — x [rows][D] bf16 -> codes [rows][D] e4m3 and
 *   scales [rows][D/32] E8M0 bytes (block i of a row covers elements
 *   32i .. 32i+31).  D % 32 == 0 (ATTN_ERR_UNSUPPORTED otherwise); with
 *   signs, each row is rotated first and D must be 128; x and codes
 *   16-byte aligned; no buffer may overlap another (ATTN_ERR_SHAPE).  Codes
 *   and scales are fixed by the rules above (bit-exact).
 */
int attn_quantize_fp8_blocks(const void *x, void *codes, uint8_t *scales, long long rows, int D,
                             const int8_t *signs, void *stream);

/*
 * attn_prefill_fp8 — attn_prefill (dense, causal or not) with the scores on
 * the FP8 matrix cores.  q, v bf16 as in attn_prefill; k8 [B][S][Hkv][128]
 * e4m3 codes and k_scale [B][S][Hkv][4] E8M0 bytes from
 * attn_quantize_fp8_blocks on K (k_scale 4-byte aligned).  Each query row is
 * multiplied by scale * log2(e) in fp32 and block-quantised by the same rule,
 * so the result is exact attention over the dequantised query (in log2 units,
 * base-2 softmax) and key, with P rounded to bf16 before P V (fp32
 * accumulation) and o bf16; lse [B][Hq][S] fp32 natural log, or NULL.
 * With signs (NULL: none), each query row is rotated as stated above before
 * it is multiplied (by scale * log2(e) / 128) and quantised, and k8 /
 * k_scale must come from attn_quantize_fp8_blocks with the same signs.
 * D must be 128, Hq/Hkv must divide 8 or be a multiple of 8.
 */
int attn_prefill_fp8(const void *q, const void *k8, const uint8_t *k_scale, const void *v, void *o,
                     float *lse, int B, int S, int Hq, int Hkv, int D, int causal, float scale,
                     const int8_t *signs, void *stream);

/*
 * attn_quantize_fp8_v — V for attn_prefill_fp8_pv: v [B][S][Hkv][128] bf16 ->
 *   v8t [B][Hkv][128][S64] e4m3 codes, dimension-major (V^T), S64 = S
 *   rounded up to a multiple of 64, keys S .. S64-1 written as code 0;
 *   v_scale [B][Hkv][S64/64][256] E8M0 bytes, one per (dim, 32 consecutive
 *   keys) by the rule above: in the 256-byte block of key tile t, byte
 *   4 * (32 * h + r) + db is the scale of dim 32 * db + r over keys
 *   64 t + 32 h .. +31 (the layout the kernel loads as is).  Codes and scales
 *   are fixed by the rule (bit-exact).  D must be 128; v, v8t 16-byte
 *   aligned; D * S64 < 2^31; no buffer may overlap another (ATTN_ERR_SHAPE).
 */
int attn_quantize_fp8_v(const void *v, void *v8t, uint8_t *v_scale, int B, int S, int Hkv, int D,
                        void *stream);

/*
 * attn_prefill_fp8_pv — attn_prefill_fp8 with P V on the FP8 matrix cores
 * too ([FA18] §18.5: both attention products on 8-bit operands with block
 * quantisation).  q, k8, k_scale as in attn_prefill_fp8; v8t, v_scale from
 * attn_quantize_fp8_v (v_scale 4-byte aligned).  Arithmetic: the scores are
 * those of attn_prefill_fp8 (log2 units); the weights P' = 2^(s - m + 3), m a
 * running reference maximum, are rounded to e4m3 (nearest even) and never
 * exceed 2^8.75 (a tile that would is first rescaled to its exact maximum);
 * O = sum P' V'' / sum P' with V'' the dequantised V and both sums over the
 * same rounded weights (fp32 accumulation); o bf16; lse [B][Hq][S] fp32
 * natural log of the row's sum of exp(scores), from the same rounded
 * weights, or NULL.  signs as in attn_prefill_fp8 (Q and K rotated, V
 * not).  D must be 128, Hq/Hkv must divide 8 or be a multiple of 8,
 * D * S64 < 2^31.
 */
int attn_prefill_fp8_pv(const void *q, const void *k8, const uint8_t *k_scale, const void *v8t,
                        const uint8_t *v_scale, void *o, float *lse, int B, int S, int Hq, int Hkv,
                        int D, int causal, float scale, const int8_t *signs, void *stream);

/*
 * rope_apply — rotary position embedding at absolute token positions, in
 * place ([ULY] §3.2 global token index table, §5.3).
 *   x [S][H][D] bf16, positions [S] int32 (device).
 * For i < D/2, theta_i = base^(-2i/D) and a = positions[t] * theta_i:
 *   x'[i]     = x[i] cos a - x[i + D/2] sin a
 *   x'[i+D/2] = x[i + D/2] cos a + x[i] sin a
 * The angle is formed and range-reduced in fp64, sin/cos and the rotation
 * run in fp32, results are rounded to bf16 (nearest-even).
 * D must be a multiple of 16 and at most 256 (ATTN_ERR_UNSUPPORTED
 * otherwise); x must be 16-byte aligned; S = 0 is a no-op.
 */
int rope_apply(void *x, const int32_t *positions, int S, int H, int D, float base, void *stream);

/*
 * rope_apply_qk — rope_apply on q [S][Hq][D] and k [S][Hkv][D] at the same
 * positions, in one launch: each token's (cos, sin) table is formed once and
 * serves its query and key heads.  Results are those of rope_apply on each
 * tensor, bit for bit.  Same rules as rope_apply; q and k must not overlap
 * (ATTN_ERR_SHAPE).
 */
int rope_apply_qk(void *q, void *k, const int32_t *positions, int S, int Hq, int Hkv, int D,
                  float base, void *stream);

/*
 * seq_to_head_permute — the local half of the Ulysses exchange ([ULY] §2.2):
 * gather this rank's heads from every sequence shard into global token order.
 *   in  [SP][S_loc][H_tot][D], out [SP*S_loc][H_tot/SP][D], elements of
 *   elem_bytes bytes (1, 2, 4 or 8), copied bit for bit:
 *   out[k*S_loc + s][h][:] = in[k][s][rank*(H_tot/SP) + h][:]
 * in and out must not overlap.
 */
int seq_to_head_permute(const void *in, void *out, int SP, int S_loc, int H_tot, int D, int rank,
                        int elem_bytes, void *stream);

/*
 * seq_to_head_permute_qkv — the same gather for the Q, K and V of one rank in
 * a single launch ([ULY] §2.2: the exchange moves all three tensors of the
 * attention input).  Q has Hq_tot heads, K and V have Hkv_tot heads; each of
 * the three is laid out and copied exactly as seq_to_head_permute describes.
 * No output may overlap any input or another output (ATTN_ERR_SHAPE).
 */
int seq_to_head_permute_qkv(const void *q_in, const void *k_in, const void *v_in, void *q_out,
                            void *k_out, void *v_out, int SP, int S_loc, int Hq_tot, int Hkv_tot,
                            int D, int rank, int elem_bytes, void *stream);

/*
 * seq_to_head_permute_qkv_rope — seq_to_head_permute_qkv for bf16 tensors with
 * RoPE applied to Q and K on the way ([ULY] §2.2 relayout; §3.2 RoPE at the
 * absolute position of each token, taken from the global token index table),
 * in one pass over memory.  positions[t] (int32, device, SP*S_loc entries) is
 * the absolute position of token t in the output's global token order.  The
 * outputs equal seq_to_head_permute_qkv followed by rope_apply on the Q and K
 * outputs, bit for bit (same rotation arithmetic; V is copied unchanged).
 * D must be a multiple of 16 and at most 256; every tensor 16-byte aligned;
 * no output may overlap any input or another output (ATTN_ERR_SHAPE).
 */
int seq_to_head_permute_qkv_rope(const void *q_in, const void *k_in, const void *v_in,
                                 void *q_out, void *k_out, void *v_out, const int32_t *positions,
                                 int SP, int S_loc, int Hq_tot, int Hkv_tot, int D, int rank,
                                 float base, void *stream);

/*
 * head_to_seq_permute — the local half of the second Ulysses exchange
 * ([ULY] §2.2; heads placed by global index as §2.3 describes): send this
 * rank's attention output back to the sequence shards.
 *   in  [SP*S_loc][H_tot/SP][D] (global token order, this rank's heads),
 *   out [SP][S_loc][H_tot][D], elements of elem_bytes bytes (1, 2, 4 or 8),
 *   copied bit for bit:
 *   out[k][s][rank*(H_tot/SP) + h][:] = in[k*S_loc + s][h][:]
 * Only this rank's head slice of out is written; the other ranks' slices are
 * left untouched, so SP calls (one per rank) assemble the full output.
 * in and out must not overlap (ATTN_ERR_SHAPE).
 */
int head_to_seq_permute(const void *in, void *out, int SP, int S_loc, int H_tot, int D, int rank,
                        int elem_bytes, void *stream);

/*
 * Context parallelism on one GPU ([MGP] §3.5: ring, striped and zigzag
 * attention; §3.5.1: round-robin-split and in-seq-split).  Block b of a split
 * into n blocks spans tokens [floor(b*S/n), floor((b+1)*S/n)) (a reading: the
 * pages only state S % N == 0 for round-robin and S >= 2N for in-seq-split).
 * A rank's tokens are listed in ascending order.
 *
 * cp_shard_tokens — number of tokens rank `rank` of N holds, or
 *   -ATTN_ERR_SHAPE / -ATTN_ERR_UNSUPPORTED if the split is not defined.
 *   Host only; touches no memory.
 */
long long cp_shard_tokens(long long S, int N, int rank, int mode);

/*
 * cp_shard — gather rank `rank`'s tokens: full [S][H][D] -> shard [n][H][D]
 *   (n = cp_shard_tokens), rows of H*D elements of elem_bytes bytes copied bit
 *   for bit, and positions[i] (int32, nullable) = global index of local token
 *   i — the global token index table of [ULY] §3.2 for this shard.
 * cp_unshard — the inverse: shard [n][H][D] back into its rows of full
 *   [S][H][D]; the other ranks' rows are left untouched.
 * Input and output must not overlap (ATTN_ERR_SHAPE).
 */
int cp_shard(const void *full, void *shard, int32_t *positions, long long S, int H, int D,
             int elem_bytes, int N, int rank, int mode, void *stream);
int cp_unshard(const void *shard, void *full, long long S, int H, int D, int elem_bytes, int N,
               int rank, int mode, void *stream);

/*
 * attn_key_limits — per-row key counts for a causal mask stated on positions
 * ([MGP] §3.5: between two ranks' shards the causal rule compares original
 * token positions):
 *   key_limit[b][i] = #{ j : k_pos[b][j] <= q_pos[b][i] }
 * q_pos [B][Sq], k_pos [B][Sk], key_limit [B][Sq], all int32 on the device.
 * k_pos must be ascending (each rank's shard is); then the allowed keys of
 * every row are a prefix of the key array, which is what
 * attn_prefill_limited consumes.
 */
int attn_key_limits(const int32_t *q_pos, const int32_t *k_pos, int32_t *key_limit, int B, int Sq,
                    int Sk, void *stream);

/*
 * attn_prefill_limited — attn_prefill (bf16, D = 128) where row i of batch b
 * attends keys [0, key_limit[b][i]) of k/v [B][Sk][Hkv][D], Sk >= 1 ([FA18] §18.3
 * online softmax over that prefix).  Limits are clamped to [0, Sk] and must
 * not decrease along i (for each b); a row with limit 0 gets O = 0 and
 * LSE = -inf, i.e. weight 0 in attn_merge.  q, o [B][Sq][Hq][D]; lse
 * [B][Hq][Sq] (nullable).  This is the partial attention of one rank's
 * queries against one key shard in ring / striped / zigzag attention.
 * accumulate = 1: o and lse (then required) already hold a normalised
 * partial of the same rows over other keys, and this call merges its own
 * partial into them in place with attn_merge's rule, so a ring of shards
 * needs no separate merge pass.
 */
int attn_prefill_limited(const void *q, const void *k, const void *v, const int32_t *key_limit,
                         void *o, float *lse, int B, int Sq, int Sk, int Hq, int Hkv, int D,
                         float scale, int accumulate, void *stream);

/*
 * attn_merge — combine two normalised partial results of the same rows over
 * disjoint key sets ([FA18] §18.3 rescale identity, as the log-sum-exp merge
 * of partial attention):
 *   M = max(La, Lb), wa = e^(La-M), wb = e^(Lb-M),
 *   O = (wa Oa + wb Ob) / (wa + wb),  LSE = M + ln(wa + wb)
 * A side with LSE = -inf has weight 0; if both do, O = 0 and LSE = -inf.
 * O* [B][S][H][D] bf16, LSE* [B][H][S] fp32 (the layouts attn_prefill
 * writes); lse is nullable.  D % 8 == 0 and D/8 divides 64.  o may be o_a or
 * o_b itself (in place), lse likewise; any other overlap is ATTN_ERR_SHAPE.
 */
int attn_merge(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b, void *o,
               float *lse, int B, int S, int H, int D, void *stream);

/* Static, human-readable text for an attn_status value. */
const char *attn_status_string(int status);

/*
 * attn_build_id — static text identifying the sources this library was
 * built from (a hash over its kernel sources, headers and compile flags), so
 * that a loader can refuse a build that does not match the sources it ships
 * with.  Never NULL; "unknown" when the build did not set it.
 */
const char *attn_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* LCAT_ATTN_H */

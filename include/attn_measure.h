/*
 * libattn measurement helper.  It is not part of the attention path and
 * computes nothing that path uses; it gives the bf16 matrix-core rate the
 * device sustains on changing operands, against which the prefill kernel's
 * throughput is read next to the published dense peak.
 */
#ifndef LCAT_ATTN_MEASURE_H
#define LCAT_ATTN_MEASURE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_measure_status {
  ATTN_MEASURE_OK = 0,
  ATTN_MEASURE_ERR_NULL = 1,  /* out is NULL */
  ATTN_MEASURE_ERR_SHAPE = 2, /* n_wg outside [1, 65536], or iters outside [4, 2^24] or not a multiple of 4 */
  ATTN_MEASURE_ERR_HIP = 7    /* the HIP runtime rejected the launch */
};

/*
 * attn_measure_mfma_rate — enqueue one launch of n_wg workgroups of 8 waves;
 * each wave issues 4 * iters v_mfma_f32_32x32x16_bf16 on uniform random bf16
 * operands in [-1, 1) held in registers (seeded by `seed`), so one launch
 * performs n_wg * 8 * iters * 4 * 32768 floating-point operations.  Each
 * workgroup reserves enough LDS to be alone on its CU.
 *   out    device float[n_wg * 512], caller-owned; receives one sum of the
 *          accumulators per thread (kept only so the products are live).
 *   stream hipStream_t as void* (NULL = default stream); the call only
 *          enqueues.  The caller times it (e.g. with events on `stream`).
 * Returns ATTN_MEASURE_OK or an error code above; argument errors are found
 * before anything is enqueued.
 */
int attn_measure_mfma_rate(float *out, int n_wg, int iters, uint32_t seed, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LCAT_ATTN_MEASURE_H */

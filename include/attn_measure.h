/*
 * libattn measurement helpers.  They are not part of the attention path and
 * compute nothing that path uses.  They give rates the device sustains, against
 * which the path's kernels are read next to the published peaks:
 *  - the bf16 matrix-core rate on changing operands (for prefill);
 *  - plain streaming HBM read and copy rates (for decode and the relayouts).
 * Conventions as in attn.h: device pointers owned by the caller, `stream` a
 * hipStream_t passed as void* (NULL = default stream), calls only enqueue,
 * argument errors are found before anything is enqueued.
 */
#ifndef LCAT_ATTN_MEASURE_H
#define LCAT_ATTN_MEASURE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_measure_status {
  ATTN_MEASURE_OK = 0,
  ATTN_MEASURE_ERR_NULL = 1,  /* a required pointer is NULL */
  ATTN_MEASURE_ERR_SHAPE = 2, /* a size outside its documented range, or overlapping buffers */
  ATTN_MEASURE_ERR_ALIGN = 4, /* a buffer is not 16-byte aligned */
  ATTN_MEASURE_ERR_HIP = 7    /* the HIP runtime rejected the launch */
};

/*
 * attn_measure_mfma_rate — enqueue one launch of n_wg workgroups of 8 waves;
 * each wave issues 4 * iters v_mfma_f32_32x32x16_bf16 on uniform random bf16
 * operands in [-1, 1) (seeded by `seed`), so one launch performs
 * n_wg * 8 * iters * 4 * 32768 floating-point operations.  Each workgroup
 * reserves enough LDS to be alone on its CU.
 *   a_from_lds  0: both operands held in registers;
 *               1: each MFMA's A operand read from LDS just before it (one
 *               16-byte read per lane per MFMA, 64 KiB of random bf16 in
 *               LDS), B from registers.  Other values: ATTN_MEASURE_ERR_SHAPE.
 *   out    device float[n_wg * 512], caller-owned; receives one sum of the
 *          accumulators per thread (kept only so the products are live).
 *   stream hipStream_t as void* (NULL = default stream); the call only
 *          enqueues.  The caller times it (e.g. with events on `stream`).
 * Returns ATTN_MEASURE_OK or an error code above; argument errors are found
 * before anything is enqueued.
 */
int attn_measure_mfma_rate(float *out, int n_wg, int iters, uint32_t seed, int a_from_lds,
                           void *stream);

/*
 * attn_measure_hbm_read — streaming read of `buf`: `waves` single-wave
 * workgroups each read one contiguous share of floor(bytes / 16 / waves)
 * 16-byte units (32 loads per lane in flight); the bytes read per launch are
 * attn_measure_hbm_read_bytes(bytes, waves).  `out` (device uint32[waves * 64])
 * receives one fold of the data per lane.  Needs waves in [1, 65536] and
 * bytes / 16 >= waves (ATTN_MEASURE_ERR_SHAPE); buf 16-byte aligned.
 */
int attn_measure_hbm_read(const void *buf, long long bytes, uint32_t *out, int waves,
                          void *stream);

/* Bytes one attn_measure_hbm_read launch reads (0 for invalid sizes). */
long long attn_measure_hbm_read_bytes(long long bytes, int waves);

/*
 * attn_measure_hbm_copy — dst[0, bytes) = src[0, bytes) with 16-byte loads
 * and non-temporal 16-byte stores, 4 per thread; bytes a positive multiple
 * of 16, both pointers 16-byte aligned.  dst == src is allowed (an in-place
 * pass: the yardstick for kernels that rewrite their input, such as
 * rope_apply); any other overlap is ATTN_MEASURE_ERR_SHAPE.
 */
int attn_measure_hbm_copy(const void *src, void *dst, long long bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LCAT_ATTN_MEASURE_H */

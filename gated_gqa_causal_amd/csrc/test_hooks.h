// test_hooks.h -- entry points of the test build of the library
// (libgatedattn_test.so, compiled with ATTN_TEST_HOOKS); the product library
// does not export them.  Only the tests load the test build.
#pragma once

#include "gatedattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Writes the prepared (normed, rotated) queries and keys the kernels use, in
 * plain layouts, for comparison with the oracle's prepared vectors.
 * qp_out: device bf16 [T - q_base][Hq][D] (may be NULL); kp_out: device bf16
 * [Hkv][T][D] (may be NULL).  Validation as attn_prefill_prefix, plus both
 * outputs NULL (ATTN_ERR_NULL_ARG) and 16-byte alignment (ATTN_ERR_ALIGN).
 */
ATTN_EXPORT int attn_debug_prepare(attn_ctx *ctx, const attn_inputs *in, int32_t T, int32_t q_base,
                                   void *qp_out, void *kp_out, void *stream);

/*
 * The fp8 cache writer's arithmetic for rows of finite values on single
 * values: q[i] = x[i] / sc[i] as the writer divides (one correctly rounded
 * reciprocal of sc, then a multiply and two FMAs) and codes[i] = the e4m3
 * code it stores for q[i].  x, sc, q: device fp32 [n]; codes: device uint8
 * [n].  The writer takes this route for rows whose largest magnitude is
 * finite and at least 2^-40 (sc >= 2^-49); other inputs are allowed and
 * give whatever the arithmetic gives.  n outside 0 .. 2^30: ATTN_ERR_RANGE;
 * a NULL pointer with n > 0: ATTN_ERR_NULL_ARG; n == 0 does nothing.
 */
ATTN_EXPORT int attn_debug_fp8_encode(const float *x, const float *sc, float *q, uint8_t *codes, int64_t n,
                                      void *stream);

#ifdef __cplusplus
}
#endif

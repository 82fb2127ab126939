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

#ifdef __cplusplus
}
#endif

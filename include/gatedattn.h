/*
 * gatedattn.h -- C ABI of the MI355X (gfx950) gated GQA causal attention
 * prefill library, libgatedattn.so.
 *
 * The operation (per query row i at absolute position p, per query head h):
 *   q, gate  = the two halves of head h's slice of the fused q|gate row;
 *   q', k'   = (1+w) RMSNorm, then rotate-half RoPE on the first 64 of 256
 *              dims from the caller's fp32 cos/sin table at the token's
 *              absolute position;
 *   s_j      = bf16(q' . k'_j) / 16 for every visible key j of KV head h/G;
 *   w        = softmax over the visible s_j (fp32), weights rounded to bf16;
 *   ctx      = bf16(sum_j w_j v_j);
 *   out      = bf16(ctx * bf16(sigmoid(gate))).
 * Key j is visible to row i iff j <= p and, in the masked entry point,
 * mask[i][j] != 0.  A row with no visible key outputs zeros.
 *
 * Sources: the QSA kernel page ("feat(qwen4): add the QSA sparse-attention
 * kernel and its golden"), sections "Summary", "What changed" and "Semantics"
 * (q|gate split, (1+w) norms, 64-of-256 partial RoPE from a shared table,
 * q.k/sqrt(256), mask polarity, fp32 softmax over bf16 scores, bf16 weights,
 * sigmoid gate before o_proj; geometry validated before sizing any buffer; an
 * empty launch is a no-op) and the attention-tile page ("cuda: widen the
 * attention query tile on sm_89 and sm_120"), review sections "Dispatch/guard"
 * and "Kernel change" (extern "C" entry points that pre-validate and return
 * errors with no silent fallback; prefix windows at an aligned q_base equal
 * the full pass), and the shared-prefix page ("run shared prompt prefixes
 * once": the rotary table is indexed by absolute position from the window
 * start).
 *
 * Conventions for every entry point:
 *   - Pointers named "device" are device memory on the context's GPU, owned
 *     by the caller; the library never frees them.  bf16 is IEEE bfloat16
 *     stored as 16-bit words.  All tensors are dense, row-major, contiguous.
 *   - Returns ATTN_OK (0) or one negative attn_status.  Arguments are fully
 *     validated on the host before any device work; a refused call leaves the
 *     device untouched.  There is no fallback path.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*,
 *     NULL = the null stream); the caller synchronises.
 *   - A context is bound to one device and owns a workspace sized at
 *     creation, so calls never allocate.  A context is not thread safe and
 *     its workspace is reused: use one context per stream.
 */
#ifndef GATEDATTN_H
#define GATEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define ATTN_EXPORT __attribute__((visibility("default")))
#else
#define ATTN_EXPORT
#endif

#define ATTN_ABI_VERSION 2
#define ATTN_HEAD_DIM 256
#define ATTN_ROTARY_DIM 64
#define ATTN_MAX_GROUP 16         /* query heads per KV head, 1..16          */
#define ATTN_MAX_TOKENS 32768     /* cap on T (keys); max_tokens <= this     */
#define ATTN_QBASE_ALIGN 128      /* q_base must be a multiple of this       */
#define ATTN_MAX_SEQS 4096        /* sequences per packed batch              */

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL_ARG = -1,   /* a required pointer is NULL                    */
    ATTN_ERR_GEOMETRY = -2,   /* unsupported head counts / dims / eps          */
    ATTN_ERR_RANGE = -3,      /* T, q_base, rows or n_pos out of range         */
    ATTN_ERR_ALIGN = -4,      /* q_base not a multiple of 128, or a pointer
                                 not 16-byte aligned                           */
    ATTN_ERR_DEVICE = -5,     /* no device, bad index, or the current device
                                 is not the context's device                   */
    ATTN_ERR_NOMEM = -6,      /* workspace allocation failed (create only)     */
    ATTN_ERR_LAUNCH = -7      /* a kernel launch or HIP runtime call failed    */
} attn_status;

typedef struct attn_ctx attn_ctx;     /* opaque */

typedef struct {
    int32_t n_q_heads;    /* Hq; a multiple of n_kv_heads                      */
    int32_t n_kv_heads;   /* Hkv >= 1; G = Hq / Hkv in 1..ATTN_MAX_GROUP       */
    int32_t head_dim;     /* must be ATTN_HEAD_DIM                             */
    int32_t rotary_dim;   /* must be ATTN_ROTARY_DIM                           */
    int32_t max_tokens;   /* 1..ATTN_MAX_TOKENS; sizes the workspace           */
    float rms_eps;        /* finite, > 0 (1e-6 for the Qwen-style models)     */
} attn_geometry;

typedef struct {
    const void *qg;        /* device bf16 [rows][Hq][2][D]: per head q then gate;
                              rows = the query rows of the call             */
    const void *k;         /* device bf16 [T][Hkv][D], raw (before norm/RoPE) */
    const void *v;         /* device bf16 [T][Hkv][D]                         */
    const void *q_norm_w;  /* device bf16 [D], applied as (1 + w)            */
    const void *k_norm_w;  /* device bf16 [D], applied as (1 + w)            */
    const float *cos_tab;  /* device fp32 [n_pos][rotary_dim/2]              */
    const float *sin_tab;  /* device fp32 [n_pos][rotary_dim/2]              */
    int32_t n_pos;         /* rows of the tables; must be >= T               */
} attn_inputs;

/* ABI version of the loaded library (ATTN_ABI_VERSION when it matches). */
ATTN_EXPORT int attn_abi_version(void);

/* Static, human-readable name of a status code; never NULL. */
ATTN_EXPORT const char *attn_status_string(int status);

/*
 * Host-only check of one call, the same one every entry point runs first.
 * kind: 0 = gated full pass (q_base must be 0), 1 = prefix window,
 * 2 = masked (q_base must be 0, mask required), 3 = bidirectional full pass
 * (q_base must be 0), 4 = append to a K/V cache (`mask` is then the cache
 * pointer: required, 16-byte aligned; k and v hold the T - q_base new rows),
 * 5 = append to an fp8 K/V cache (as 4, with the fp8 cache).
 * T keys, query rows T - q_base.  Touches no device; usable without a GPU.
 */
ATTN_EXPORT int attn_validate(const attn_geometry *geom, const attn_inputs *in, int32_t T, int32_t q_base,
                  int32_t kind, const void *mask, const void *out);

/*
 * Creates a context on `device` for `geom`, allocating its workspace (about
 * 2 * Hkv * max_tokens * D * 2 bytes for prepared keys and values, plus
 * max_tokens^2 / 8 bytes of packed mask bits, max_tokens * Hq * 8 bytes
 * of softmax row statistics, and small device and pinned host tables for
 * packed batches and the attention kernel's work schedule).  The device becomes current
 * on the calling thread.  On success *out holds the context; on failure
 * *out is NULL and nothing stays allocated.  The context keeps the work
 * schedule of its last launch shape (tokens, q_base, masked or not): a call
 * with another shape plans a new one on the host first (tens of
 * microseconds; packed batches plan on every call).
 */
ATTN_EXPORT int attn_ctx_create(const attn_geometry *geom, int device, attn_ctx **out);

/* Frees the context and its workspace.  NULL is a no-op.  Not stream-ordered:
   the caller must have synchronised work that uses the context. */
ATTN_EXPORT void attn_ctx_destroy(attn_ctx *ctx);

/*
 * Dense causal full pass over S tokens: query rows = keys = positions 0..S-1.
 * out: device bf16 [S][Hq * D] (head-major within a row: the o_proj input).
 * S == 0 is a no-op returning ATTN_OK.
 */
ATTN_EXPORT int attn_prefill_gated(attn_ctx *ctx, const attn_inputs *in, int32_t S, void *out, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the dense
 * causal full pass of attn_prefill_gated without a context.  Same inputs,
 * layouts and output, bit for bit; geom describes the call (S <= max_tokens).
 * The prepared keys and transposed values go to a fixed scratch array in the
 * library's device code, ATTN_NOALLOC_SCRATCH_BYTES per device, held by every
 * device the library runs on until the process ends; the first call on a
 * device looks its address up once (with that device current).  The call
 * allocates nothing.  Limit: 2 * n_kv_heads * round_up(S, 64) * 256 * 2 bytes
 * <= ATTN_NOALLOC_SCRATCH_BYTES (n_kv_heads * round_up(S, 64) <= 32768, e.g.
 * 4 KV heads at 8192 tokens), else ATTN_ERR_RANGE before any device work.
 * Errors as attn_prefill_gated, plus ATTN_ERR_DEVICE if the current device
 * cannot be queried.  Every call on one device shares that device's scratch:
 * calls that overlap on one device (other streams, other threads) race and
 * must be ordered by the caller.  S == 0 is a no-op.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
ATTN_EXPORT int attn_prefill_gated_noalloc(const attn_geometry *geom, const attn_inputs *in, int32_t S, void *out,
                                           void *stream);

/*
 * Prefix-continuation window: keys at positions 0..T-1, query rows at
 * positions q_base..T-1 (qg holds T - q_base rows; out is device bf16
 * [T - q_base][Hq * D]).  q_base must be a multiple of ATTN_QBASE_ALIGN and
 * <= T; q_base == T is a no-op.  Each output row equals, bit for bit, the
 * same row of attn_prefill_gated over all T tokens.
 */
ATTN_EXPORT int attn_prefill_prefix(attn_ctx *ctx, const attn_inputs *in, int32_t T, int32_t q_base,
                        void *out, void *stream);

/*
 * Masked full pass over S tokens: key j is visible to row i iff j <= i and
 * mask[i * S + j] != 0.  mask: device uint8 [S][S] (any alignment).
 * Key tiles hidden for a whole block of rows are skipped.  With an
 * all-visible mask the output equals attn_prefill_gated bit for bit.
 */
ATTN_EXPORT int attn_prefill_masked(attn_ctx *ctx, const attn_inputs *in, int32_t S, const uint8_t *mask,
                        void *out, void *stream);

/*
 * Bidirectional full pass over S tokens (no causal predicate: every row
 * sees keys 0..S-1), the variant the system1-omni gated-attention page
 * ("cuda: widen the attention query tile on sm_89 and sm_120") runs for the
 * vision path through the same launch.  Same inputs, layouts and errors as
 * attn_prefill_gated; out: device bf16 [S][Hq * D].  S == 0 is a no-op.
 * The last row equals attn_prefill_gated's last row bit for bit.
 */
ATTN_EXPORT int attn_prefill_bidirectional(attn_ctx *ctx, const attn_inputs *in, int32_t S, void *out,
                                           void *stream);

/*
 * Attention weights (the QSA kernel page, "What changed" and its timing
 * table: the kernel also writes the normalised weights, bf16 [rows][heads]
 * [tokens], which its golden checks).  Runs the pass of `kind` (0 gated,
 * 1 prefix window, 2 masked with `mask`, 3 bidirectional; the K/V cache kinds
 * are refused with ATTN_ERR_RANGE) exactly as its own entry point does (same
 * arguments, limits and `out`, bit for bit), then writes
 *   weights[i][h][j] = bf16(exp(s_ij - m_ih) / l_ih)
 * into the caller's device buffer `weights`, bf16 [T - q_base][Hq][T],
 * 16-byte aligned: s_ij = bf16(q_i . k_j) / 16 is row i's rounded score,
 * m_ih and l_ih the reference max and the sum of the bf16 weight numerators
 * the pass's online softmax ended with, so that out's context is
 * sum_j weight * v_j up to the rounding of the weights.  Hidden keys (causal,
 * masked, or a row with no visible key) give 0; every element is written.
 * Row statistics live in the context's workspace (max_tokens * Hq * 8
 * bytes), so calls on one context must be stream-ordered.
 * attn_validate_weights runs the host-only checks: attn_validate's, then
 * weights non-NULL (ATTN_ERR_NULL_ARG) and 16-byte aligned (ATTN_ERR_ALIGN);
 * an empty window is a no-op and skips them.
 */
ATTN_EXPORT int attn_validate_weights(const attn_geometry *geom, const attn_inputs *in, int32_t T,
                                      int32_t q_base, int32_t kind, const void *mask, const void *out,
                                      const void *weights);
ATTN_EXPORT int attn_prefill_weights(attn_ctx *ctx, const attn_inputs *in, int32_t T, int32_t q_base,
                                     int32_t kind, const uint8_t *mask, void *out, void *weights,
                                     void *stream);

/*
 * Cached prefix continuation (the prefix state of the system1-omni
 * "run shared prompt prefixes once" page keeps a prefix's K/V per
 * attention layer).  A caller-owned device buffer of attn_kv_cache_bytes()
 * holds prepared (normed, rotated) keys and transposed values in the
 * library's tile layout for one geometry (max_tokens positions).
 *
 * attn_prefill_append: positions q_base..T-1 are new.  in->k and in->v hold
 * their raw rows only (bf16 [T - q_base][Hkv][D]); qg holds their query rows
 * ([T - q_base][Hq][2][D]).  The call prepares the new keys into the cache,
 * then computes the query rows q_base..T-1 over cache keys 0..T-1, whose
 * positions 0..q_base-1 earlier calls on the same cache prepared.  q_base
 * must be a multiple of ATTN_QBASE_ALIGN; q_base == 0 starts a cache.
 * out: bf16 [T - q_base][Hq * D].  Each row equals, bit for bit, the same row
 * of attn_prefill_gated over all T tokens.  Calls on one cache must be
 * stream-ordered; T - q_base == 0 is a no-op.
 */
ATTN_EXPORT int attn_kv_cache_bytes(const attn_geometry *geom, size_t *bytes);
ATTN_EXPORT int attn_prefill_append(attn_ctx *ctx, const attn_inputs *in, int32_t T, int32_t q_base,
                                    void *kv_cache, void *out, void *stream);

/*
 * fp8 K/V cache (the long-prompt prefill page, Kernels list: e4m3 cache rows
 * with an fp32 scale each, widened to bf16 for the attention products).
 * Layout of the caller-owned buffer (attn_kv_cache_fp8_bytes bytes, 16-byte
 * aligned), with tpad = max_tokens rounded up to 64 and rows = positions:
 *   uint8 key rows   [Hkv][tpad][256]   prepared (normed, rotated) keys, e4m3
 *   uint8 value rows [Hkv][tpad][256]   raw values, e4m3
 *   fp32 key scales  [Hkv][tpad]        one per key row
 *   fp32 value scales[Hkv][tpad]        one per value row
 * E4M3 is the OCP 8-bit floating point format (bias 7, no infinities, 448
 * the largest finite magnitude).  A row's scale is amax / 448 (1 for an all
 * zero row, and for a row holding a NaN, whose amax is NaN); each value is
 * encoded from value / scale (fp32 division, correctly rounded) to the
 * nearest code, ties to the even mantissa, magnitudes past 448 saturated,
 * NaN to 0x7F; the attention
 * uses bf16(code value * scale).  attn_prefill_append_fp8 works as
 * attn_prefill_append (same arguments, alignment and limits): it encodes the
 * rows of positions q_base..T-1 into the cache, widens rows 0..T-1 into the
 * context's workspace, and runs the window's rows over keys 0..T-1.  Chunked
 * appends give the single call's output bit for bit.
 */
ATTN_EXPORT int attn_kv_cache_fp8_bytes(const attn_geometry *geom, size_t *bytes);
ATTN_EXPORT int attn_prefill_append_fp8(attn_ctx *ctx, const attn_inputs *in, int32_t T, int32_t q_base,
                                        void *kv_cache8, void *out, void *stream);

/*
 * Packed batch of independent sequences in one launch (the serving page's
 * batched gated attention: a pack of candidates must give each candidate the
 * bits it gets alone, whatever its neighbours and their order).
 * seq_lens: host int32 [n_seqs], read during the call only.  Rows of qg, k, v
 * and out hold the sequences back to back: sequence i starts at row
 * sum_{j<i} seq_lens[j] (qg [total][Hq][2][D], k and v [total][Hkv][D], out
 * [total][Hq * D]).  Each sequence is a dense causal pass at positions
 * 0..len-1 (cos/sin rows 0..len-1, so n_pos >= the longest length), sharing
 * the norm weights; its output rows equal attn_prefill_gated on that
 * sequence alone, bit for bit.  Limits: 0 <= n_seqs <= ATTN_MAX_SEQS, every
 * length in [0, max_tokens], the total <= max_tokens, and the sum of the
 * lengths rounded up to 32 <= max_tokens rounded up to 64 (each sequence's
 * keys start on a 32-key tile of the workspace), else ATTN_ERR_RANGE.
 * Zero-length sequences are allowed; a total of 0 is a no-op.  The call
 * copies a small table (sequences, tiles, row blocks) to the device through
 * the context's pinned staging buffer, waiting first for the previous batch
 * call's copy on the context to land.  attn_validate_batch runs the same
 * host-only checks.
 */
ATTN_EXPORT int attn_validate_batch(const attn_geometry *geom, const attn_inputs *in, int32_t n_seqs,
                                    const int32_t *seq_lens, const void *out);
ATTN_EXPORT int attn_prefill_gated_batch(attn_ctx *ctx, const attn_inputs *in, int32_t n_seqs,
                                         const int32_t *seq_lens, void *out, void *stream);

/*
 * Branches of one shared prefix, packed into one launch (the serving page's
 * shared-prefix batched gated attention; on the shared-prefix page a common
 * prefix is computed a single time and each branch then resumes from the state
 * it left, its tokens placed after the prefix and still causal).  kv_cache: a
 * caller-owned cache of this context's geometry (attn_kv_cache_bytes) whose
 * positions 0..prefix_len-1 earlier attn_prefill_append calls prepared; this
 * call only reads it.
 * branch_lens: host int32 [n_branches], read during the call only.  Rows of
 * qg, k, v and out hold the branches' new tokens back to back, as in
 * attn_prefill_gated_batch.  Branch b's tokens sit at positions prefix_len ..
 * prefix_len + len_b - 1 (cos/sin rows by position, so n_pos >= prefix_len +
 * the longest branch); its queries attend to the prefix's keys and to its own
 * keys up to their position, never to another branch's.  Its own keys are
 * prepared into the context's workspace, not into the cache.  Its output rows
 * equal, bit for bit, attn_prefill_append with q_base = prefix_len on a copy of
 * the cache holding that branch alone, and so the rows prefix_len.. of
 * attn_prefill_gated over the prefix and that branch.  prefix_len must be a
 * multiple of ATTN_QBASE_ALIGN (else ATTN_ERR_ALIGN) with prefix_len + every
 * length <= max_tokens; the branch lengths follow attn_prefill_gated_batch's
 * limits (else ATTN_ERR_RANGE).  prefix_len == 0 is a plain packed batch (the
 * cache is then unused and may be NULL; otherwise NULL gives
 * ATTN_ERR_NULL_ARG, a pointer off 16 bytes ATTN_ERR_ALIGN); a total of 0 new
 * tokens is a no-op.  The table goes through the same staging buffer as a
 * packed batch.  attn_validate_shared_batch runs the same host-only checks.
 */
ATTN_EXPORT int attn_validate_shared_batch(const attn_geometry *geom, const attn_inputs *in, int32_t prefix_len,
                                           const void *kv_cache, int32_t n_branches, const int32_t *branch_lens,
                                           const void *out);
ATTN_EXPORT int attn_prefill_shared_batch(attn_ctx *ctx, const attn_inputs *in, int32_t prefix_len,
                                          const void *kv_cache, int32_t n_branches, const int32_t *branch_lens,
                                          void *out, void *stream);

/*
 * Per-kernel timing with HIP events recorded on the call's stream around
 * each launch.  enable != 0 creates an event pool (outside any timed
 * region) and starts recording for every kernel; 0 stops.
 * attn_ctx_set_timing_mask does the same for the kernels whose bits
 * (1 << ATTN_KERNEL_*) are set in kernel_mask (0 stops; bits outside
 * ATTN_TIMING_ALL: ATTN_ERR_RANGE): each recorded event costs the stream a
 * few microseconds, so a caller timing whole calls records only the kernels
 * it needs.  attn_ctx_read_timing waits for the recorded events, returns the
 * summed duration (ms) and launch count of one kernel since the last read,
 * and clears them.  kernel: ATTN_KERNEL_*.  Errors: ATTN_ERR_NULL_ARG,
 * ATTN_ERR_DEVICE (another device current), ATTN_ERR_NOMEM (event pool).
 */
#define ATTN_KERNEL_KV_PROLOGUE 0
#define ATTN_KERNEL_MASK_PACK 1
#define ATTN_KERNEL_ATTENTION 2
#define ATTN_KERNEL_WEIGHTS 3
#define ATTN_TIMING_ALL 15                /* the four kernels above */
ATTN_EXPORT int attn_ctx_set_timing(attn_ctx *ctx, int enable);
ATTN_EXPORT int attn_ctx_set_timing_mask(attn_ctx *ctx, int kernel_mask);
ATTN_EXPORT int attn_ctx_read_timing(attn_ctx *ctx, int kernel, double *total_ms, int32_t *launches);

/*
 * Calibration (not part of the attention path): the bf16 matrix-core rate the
 * current device sustains under its power limit.  Launches one workgroup per
 * compute unit on `stream`, one wave per SIMD issuing back-to-back
 * v_mfma_f32_32x32x16_bf16 (iters x 16 per wave) on pseudo-random operands,
 * waits for it, and returns the mean shader clock (MHz, s_memtime cycles over
 * s_memrealtime's 100 MHz ticks) and the MFMA rate (TFLOP/s).  Allocates and
 * frees a few KB of device memory itself; blocking.  iters in [1, 1e7], else
 * ATTN_ERR_RANGE.
 */
ATTN_EXPORT int attn_mfma_clock_probe(int32_t iters, void *stream, double *mhz, double *tflops);

#ifdef __cplusplus
}
#endif

#endif /* GATEDATTN_H */

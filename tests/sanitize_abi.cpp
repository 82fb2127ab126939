// Host-side checks of the C ABI under AddressSanitizer and UBSan (host code
// only; the device code is compiled as usual and never launched): every
// refusal path of the validation, the batch planner, the size queries and the
// null-context entry points, with the status each must return.  No call here
// reaches a device.  Exit status 0 when every check holds.
#include "gatedattn.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

static int failures = 0;
#define EXPECT(call, want)                                                                          \
    do {                                                                                            \
        const int got_ = (call);                                                                    \
        if (got_ != (want)) {                                                                       \
            ++failures;                                                                             \
            std::printf("FAIL line %d: %s -> %d, expected %d\n", __LINE__, #call, got_, (int)(want)); \
        }                                                                                           \
    } while (0)

static attn_geometry geom(int hq = 24, int hkv = 2, int max_tokens = 256, float eps = 1e-6f)
{
    return attn_geometry{hq, hkv, ATTN_HEAD_DIM, ATTN_ROTARY_DIM, max_tokens, eps};
}

int main()
{
    // Buffers the validation looks at (never dereferenced): 16-byte aligned,
    // and one byte off for the alignment refusals.
    alignas(16) static unsigned char buf[64];
    void *A = buf, *M = buf + 1;
    const float *FA = reinterpret_cast<const float *>(buf);
    const float *FM = reinterpret_cast<const float *>(buf + 1);
    attn_inputs in{A, A, A, A, A, FA, FA, 256};

    for (int s = -12; s <= 2; ++s)
        if (!attn_status_string(s) || !std::strlen(attn_status_string(s)))
            ++failures;
    EXPECT(attn_abi_version(), ATTN_ABI_VERSION);

    // geometry
    attn_geometry g = geom();
    EXPECT(attn_validate(nullptr, &in, 64, 0, 0, nullptr, A), ATTN_ERR_NULL_ARG);
    attn_geometry b = g; b.head_dim = 128;       EXPECT(attn_validate(&b, &in, 64, 0, 0, nullptr, A), ATTN_ERR_GEOMETRY);
    b = g; b.rotary_dim = 32;                    EXPECT(attn_validate(&b, &in, 64, 0, 0, nullptr, A), ATTN_ERR_GEOMETRY);
    b = g; b.n_kv_heads = 0;                     EXPECT(attn_validate(&b, &in, 64, 0, 0, nullptr, A), ATTN_ERR_GEOMETRY);
    b = g; b.n_kv_heads = 5;                     EXPECT(attn_validate(&b, &in, 64, 0, 0, nullptr, A), ATTN_ERR_GEOMETRY);
    b = geom(34, 2);                             EXPECT(attn_validate(&b, &in, 64, 0, 0, nullptr, A), ATTN_ERR_GEOMETRY);
    b = geom(1025 * 2, 1025);                    EXPECT(attn_validate(&b, &in, 64, 0, 0, nullptr, A), ATTN_ERR_GEOMETRY);
    b = geom(INT32_MAX, 1);                      EXPECT(attn_validate(&b, &in, 64, 0, 0, nullptr, A), ATTN_ERR_GEOMETRY);
    b = g; b.rms_eps = 0.0f;                     EXPECT(attn_validate(&b, &in, 64, 0, 0, nullptr, A), ATTN_ERR_GEOMETRY);
    b = g; b.rms_eps = NAN;                      EXPECT(attn_validate(&b, &in, 64, 0, 0, nullptr, A), ATTN_ERR_GEOMETRY);
    b = g; b.rms_eps = INFINITY;                 EXPECT(attn_validate(&b, &in, 64, 0, 0, nullptr, A), ATTN_ERR_GEOMETRY);
    b = g; b.max_tokens = 0;                     EXPECT(attn_validate(&b, &in, 0, 0, 0, nullptr, A), ATTN_ERR_RANGE);
    b = g; b.max_tokens = ATTN_MAX_TOKENS + 1;   EXPECT(attn_validate(&b, &in, 64, 0, 0, nullptr, A), ATTN_ERR_RANGE);

    // ranges, kinds, alignment, pointers
    EXPECT(attn_validate(&g, &in, 64, 0, -1, nullptr, A), ATTN_ERR_RANGE);
    EXPECT(attn_validate(&g, &in, 64, 0, 6, nullptr, A), ATTN_ERR_RANGE);
    EXPECT(attn_validate(&g, &in, -1, 0, 0, nullptr, A), ATTN_ERR_RANGE);
    EXPECT(attn_validate(&g, &in, 257, 0, 0, nullptr, A), ATTN_ERR_RANGE);
    EXPECT(attn_validate(&g, &in, INT32_MIN, 0, 1, nullptr, A), ATTN_ERR_RANGE);
    EXPECT(attn_validate(&g, &in, 200, -128, 1, nullptr, A), ATTN_ERR_RANGE);
    EXPECT(attn_validate(&g, &in, 200, 256, 1, nullptr, A), ATTN_ERR_RANGE);
    for (int kind : {0, 2, 3})
        EXPECT(attn_validate(&g, &in, 200, 128, kind, A, A), ATTN_ERR_RANGE);
    EXPECT(attn_validate(&g, &in, 200, 64, 1, nullptr, A), ATTN_ERR_ALIGN);
    EXPECT(attn_validate(&g, &in, 128, 128, 1, nullptr, nullptr), ATTN_OK);     // empty window
    EXPECT(attn_validate(&g, nullptr, 0, 0, 0, nullptr, nullptr), ATTN_OK);      // empty launch
    EXPECT(attn_validate(&g, nullptr, 64, 0, 0, nullptr, A), ATTN_ERR_NULL_ARG);
    EXPECT(attn_validate(&g, &in, 64, 0, 0, nullptr, nullptr), ATTN_ERR_NULL_ARG);
    for (int f = 0; f < 7; ++f) {
        attn_inputs x = in;
        const void **fields[] = {&x.qg, &x.k, &x.v, &x.q_norm_w, &x.k_norm_w};
        if (f < 5) *fields[f] = nullptr; else if (f == 5) x.cos_tab = nullptr; else x.sin_tab = nullptr;
        EXPECT(attn_validate(&g, &x, 64, 0, 0, nullptr, A), ATTN_ERR_NULL_ARG);
        if (f < 5) *fields[f] = M; else if (f == 5) x.cos_tab = FM; else x.sin_tab = FM;
        EXPECT(attn_validate(&g, &x, 64, 0, 0, nullptr, A), ATTN_ERR_ALIGN);
    }
    EXPECT(attn_validate(&g, &in, 64, 0, 0, nullptr, M), ATTN_ERR_ALIGN);
    for (int kind : {2, 4, 5})
        EXPECT(attn_validate(&g, &in, 64, 0, kind, nullptr, A), ATTN_ERR_NULL_ARG);
    EXPECT(attn_validate(&g, &in, 64, 0, 2, M, A), ATTN_OK);                    // a mask may be unaligned
    EXPECT(attn_validate(&g, &in, 64, 0, 4, M, A), ATTN_ERR_ALIGN);             // a cache may not
    attn_inputs shortt = in; shortt.n_pos = 63;
    EXPECT(attn_validate(&g, &shortt, 64, 0, 0, nullptr, A), ATTN_ERR_RANGE);

    // weights
    EXPECT(attn_validate_weights(nullptr, &in, 64, 0, 0, nullptr, A, A), ATTN_ERR_NULL_ARG);
    EXPECT(attn_validate_weights(&g, &in, 64, 0, 4, A, A, A), ATTN_ERR_RANGE);
    EXPECT(attn_validate_weights(&g, &in, 64, 0, 0, nullptr, A, nullptr), ATTN_ERR_NULL_ARG);
    EXPECT(attn_validate_weights(&g, &in, 64, 0, 0, nullptr, A, M), ATTN_ERR_ALIGN);
    EXPECT(attn_validate_weights(&g, &in, 0, 0, 0, nullptr, nullptr, nullptr), ATTN_OK);
    EXPECT(attn_validate_weights(&g, &in, 64, 0, 0, nullptr, A, A), ATTN_OK);

    // packed batches
    attn_geometry gb = geom(24, 2, 1024);
    std::vector<int32_t> lens = {100, 0, 33, 200};
    EXPECT(attn_validate_batch(&gb, &in, -1, lens.data(), A), ATTN_ERR_RANGE);
    EXPECT(attn_validate_batch(&gb, &in, ATTN_MAX_SEQS + 1, lens.data(), A), ATTN_ERR_RANGE);
    EXPECT(attn_validate_batch(&gb, &in, 4, nullptr, A), ATTN_ERR_NULL_ARG);
    EXPECT(attn_validate_batch(&gb, &in, 0, nullptr, nullptr), ATTN_OK);
    EXPECT(attn_validate_batch(&gb, &in, 4, lens.data(), A), ATTN_OK);
    lens[2] = -1;   EXPECT(attn_validate_batch(&gb, &in, 4, lens.data(), A), ATTN_ERR_RANGE);
    lens[2] = 1025; EXPECT(attn_validate_batch(&gb, &in, 4, lens.data(), A), ATTN_ERR_RANGE);
    lens[2] = INT32_MAX; EXPECT(attn_validate_batch(&gb, &in, 4, lens.data(), A), ATTN_ERR_RANGE);
    std::vector<int32_t> many(ATTN_MAX_SEQS, 1024);                          // sum far past the cap
    EXPECT(attn_validate_batch(&gb, &in, ATTN_MAX_SEQS, many.data(), A), ATTN_ERR_RANGE);
    std::vector<int32_t> tiles(33, 1);                                       // 33 tiles of 32 > tpad 1024
    EXPECT(attn_validate_batch(&gb, &in, 33, tiles.data(), A), ATTN_ERR_RANGE);
    std::vector<int32_t> zeros(ATTN_MAX_SEQS, 0);
    EXPECT(attn_validate_batch(&gb, &in, ATTN_MAX_SEQS, zeros.data(), nullptr), ATTN_OK);
    lens = {100, 0, 33, 200};
    attn_inputs shortb = in; shortb.n_pos = 199;
    EXPECT(attn_validate_batch(&gb, &shortb, 4, lens.data(), A), ATTN_ERR_RANGE);
    EXPECT(attn_validate_batch(&gb, &in, 4, lens.data(), M), ATTN_ERR_ALIGN);
    EXPECT(attn_prefill_gated_batch(nullptr, &in, 4, lens.data(), A, nullptr), ATTN_ERR_NULL_ARG);

    // branches of a shared prefix (lens 100, 0, 33, 200 after a 512-token prefix)
    attn_inputs longb = in; longb.n_pos = 1024;
    EXPECT(attn_validate_shared_batch(&gb, &longb, 512, A, 4, lens.data(), A), ATTN_OK);
    EXPECT(attn_validate_shared_batch(&gb, &longb, 0, nullptr, 4, lens.data(), A), ATTN_OK);
    EXPECT(attn_validate_shared_batch(&gb, &longb, 64, A, 4, lens.data(), A), ATTN_ERR_ALIGN);
    EXPECT(attn_validate_shared_batch(&gb, &longb, -128, A, 4, lens.data(), A), ATTN_ERR_RANGE);
    EXPECT(attn_validate_shared_batch(&gb, &longb, INT32_MIN, A, 4, lens.data(), A), ATTN_ERR_RANGE);
    EXPECT(attn_validate_shared_batch(&gb, &longb, 1152, A, 4, lens.data(), A), ATTN_ERR_RANGE);
    EXPECT(attn_validate_shared_batch(&gb, &longb, 896, A, 4, lens.data(), A), ATTN_ERR_RANGE);  // 896 + 200
    EXPECT(attn_validate_shared_batch(&gb, &longb, 512, nullptr, 4, lens.data(), A), ATTN_ERR_NULL_ARG);
    EXPECT(attn_validate_shared_batch(&gb, &longb, 512, M, 4, lens.data(), A), ATTN_ERR_ALIGN);
    EXPECT(attn_validate_shared_batch(&gb, &longb, 512, A, 4, nullptr, A), ATTN_ERR_NULL_ARG);
    EXPECT(attn_validate_shared_batch(&gb, &longb, 512, A, ATTN_MAX_SEQS + 1, lens.data(), A), ATTN_ERR_RANGE);
    EXPECT(attn_validate_shared_batch(&gb, &longb, 512, A, 0, nullptr, nullptr), ATTN_OK);
    EXPECT(attn_validate_shared_batch(&gb, &longb, 512, A, ATTN_MAX_SEQS, zeros.data(), nullptr), ATTN_OK);
    EXPECT(attn_validate_shared_batch(&gb, &longb, 512, A, ATTN_MAX_SEQS, many.data(), A), ATTN_ERR_RANGE);
    longb.n_pos = 711;
    EXPECT(attn_validate_shared_batch(&gb, &longb, 512, A, 4, lens.data(), A), ATTN_ERR_RANGE);
    EXPECT(attn_validate_shared_batch(nullptr, &in, 512, A, 4, lens.data(), A), ATTN_ERR_NULL_ARG);
    EXPECT(attn_prefill_shared_batch(nullptr, &in, 512, A, 4, lens.data(), A, nullptr), ATTN_ERR_NULL_ARG);

    // size queries
    size_t bytes = 1;
    EXPECT(attn_kv_cache_bytes(&g, nullptr), ATTN_ERR_NULL_ARG);
    b = g; b.n_kv_heads = 5;
    EXPECT(attn_kv_cache_bytes(&b, &bytes), ATTN_ERR_GEOMETRY);
    EXPECT((int)bytes, 0);
    EXPECT(attn_kv_cache_bytes(&g, &bytes), ATTN_OK);
    EXPECT(bytes == (size_t)2 * 2 * 256 * ATTN_HEAD_DIM * 2, true);
    EXPECT(attn_kv_cache_fp8_bytes(&g, &bytes), ATTN_OK);
    EXPECT(bytes == (size_t)2 * 2 * 256 * ATTN_HEAD_DIM + (size_t)2 * 2 * 256 * 4, true);
    attn_geometry gmax = geom(16, 16, ATTN_MAX_TOKENS);
    EXPECT(attn_kv_cache_bytes(&gmax, &bytes), ATTN_OK);

    // the allocation-free entry point: host refusals only
    attn_geometry g4 = geom(16, 4, ATTN_MAX_TOKENS);
    attn_inputs big = in; big.n_pos = ATTN_MAX_TOKENS;
    EXPECT(attn_prefill_gated_noalloc(&g4, &big, 8193, A, nullptr), ATTN_ERR_RANGE);
    EXPECT(attn_prefill_gated_noalloc(&g4, &big, ATTN_MAX_TOKENS, A, nullptr), ATTN_ERR_RANGE);
    EXPECT(attn_prefill_gated_noalloc(&g, &in, 257, A, nullptr), ATTN_ERR_RANGE);
    EXPECT(attn_prefill_gated_noalloc(nullptr, &in, 64, A, nullptr), ATTN_ERR_NULL_ARG);
    EXPECT(attn_prefill_gated_noalloc(&g, nullptr, 64, A, nullptr), ATTN_ERR_NULL_ARG);
    EXPECT(attn_prefill_gated_noalloc(&g, &in, 0, nullptr, nullptr), ATTN_OK);

    // contexts: refusals before any device call; null contexts
    attn_ctx *ctx = reinterpret_cast<attn_ctx *>(0x1);
    EXPECT(attn_ctx_create(&g, 0, nullptr), ATTN_ERR_NULL_ARG);
    b = g; b.n_kv_heads = 5;
    EXPECT(attn_ctx_create(&b, 0, &ctx), ATTN_ERR_GEOMETRY);
    EXPECT(ctx == nullptr, true);
    b = g; b.max_tokens = 0;
    EXPECT(attn_ctx_create(&b, 0, &ctx), ATTN_ERR_RANGE);
    EXPECT(attn_prefill_gated(nullptr, &in, 64, A, nullptr), ATTN_ERR_NULL_ARG);
    EXPECT(attn_prefill_prefix(nullptr, &in, 256, 128, A, nullptr), ATTN_ERR_NULL_ARG);
    EXPECT(attn_prefill_masked(nullptr, &in, 64, static_cast<const uint8_t *>(A), A, nullptr), ATTN_ERR_NULL_ARG);
    EXPECT(attn_prefill_bidirectional(nullptr, &in, 64, A, nullptr), ATTN_ERR_NULL_ARG);
    EXPECT(attn_prefill_append(nullptr, &in, 256, 128, A, A, nullptr), ATTN_ERR_NULL_ARG);
    EXPECT(attn_prefill_append_fp8(nullptr, &in, 256, 128, A, A, nullptr), ATTN_ERR_NULL_ARG);
    EXPECT(attn_prefill_weights(nullptr, &in, 64, 0, 0, nullptr, A, A, nullptr), ATTN_ERR_NULL_ARG);
    EXPECT(attn_ctx_set_timing(nullptr, 1), ATTN_ERR_NULL_ARG);
    EXPECT(attn_ctx_set_timing_mask(nullptr, 1), ATTN_ERR_NULL_ARG);
    double ms = 0.0;
    int32_t n = 0;
    EXPECT(attn_ctx_read_timing(nullptr, 0, &ms, &n), ATTN_ERR_NULL_ARG);
    double mhz = 0.0, tf = 0.0;
    EXPECT(attn_mfma_clock_probe(100, nullptr, nullptr, &tf), ATTN_ERR_NULL_ARG);
    EXPECT(attn_mfma_clock_probe(0, nullptr, &mhz, &tf), ATTN_ERR_RANGE);
    attn_ctx_destroy(nullptr);

    std::printf("%s (%d failures)\n", failures ? "FAILED" : "abi host checks ok", failures);
    return failures ? 1 : 0;
}

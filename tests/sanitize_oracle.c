/*
 * The CPU oracle under AddressSanitizer and UBSan: oracle.c is compiled into
 * this driver as one translation unit, and every entry point runs on edge
 * shapes (one token, ragged lengths, a prefix window, a mask with fully hidden
 * rows, the bidirectional pass, every optional output) with buffers of exactly
 * the documented sizes, plus the refusals (short table, rows out of range,
 * a head count that does not divide).  Exit status 0 when every call returns
 * what it must; any out-of-bounds access or undefined behaviour aborts.
 */
#include "../oracle/oracle.c"

#include <stdio.h>

static int failures = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            ++failures;                                                     \
            printf("FAIL line %d: %s\n", __LINE__, #cond);                  \
        }                                                                   \
    } while (0)

static uint32_t rng = 12345u;
static float unif(void)
{
    rng = rng * 1664525u + 1013904223u;
    return (float)(rng >> 8) / 16777216.0f * 2.0f - 1.0f;
}

static bf16_t *bf16_buf(size_t n, float scale)
{
    bf16_t *p = (bf16_t *)malloc(sizeof(bf16_t) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i)
        p[i] = f32_to_bf16(unif() * scale);
    return p;
}

static float *table(int n_pos, int half, int is_sin)
{
    float *t = (float *)malloc(sizeof(float) * (size_t)n_pos * half);
    for (int p = 0; p < n_pos; ++p)
        for (int j = 0; j < half; ++j) {
            const double a = p * pow(1e7, -2.0 * j / (2.0 * half));
            t[(size_t)p * half + j] = (float)(is_sin ? sin(a) : cos(a));
        }
    return t;
}

static void run_case(int T, int Hq, int Hkv, int q_base, int masked, int causal)
{
    const int D = 256, R = 64, rows = T - q_base;
    oracle_problem p;
    memset(&p, 0, sizeof p);
    p.n_q_heads = Hq;
    p.n_kv_heads = Hkv;
    p.head_dim = D;
    p.rotary_dim = R;
    p.rms_eps = 1e-6f;
    p.T = T;
    p.q_base = q_base;
    p.causal = causal;
    p.score_f64 = T & 1;      /* both readings of the score's dot product */
    bf16_t *qg = bf16_buf((size_t)rows * Hq * 2 * D, 2.0f);
    bf16_t *k = bf16_buf((size_t)T * Hkv * D, 2.0f);
    bf16_t *v = bf16_buf((size_t)T * Hkv * D, 2.0f);
    bf16_t *wq = bf16_buf(D, 0.2f), *wk = bf16_buf(D, 0.2f);
    float *ct = table(T, R / 2, 0), *st = table(T, R / 2, 1);
    uint8_t *mask = NULL;
    if (masked) {
        mask = (uint8_t *)malloc((size_t)rows * T);
        for (size_t i = 0; i < (size_t)rows * T; ++i)
            mask[i] = unif() > 0.5f;
        memset(mask, 0, (size_t)T);                   /* row 0: nothing visible */
        if (rows > 3)
            memset(mask + (size_t)3 * T, 0, (size_t)T);
    }
    p.qg = qg; p.k = k; p.v = v; p.q_norm_w = wq; p.k_norm_w = wk;
    p.cos_tab = ct; p.sin_tab = st; p.n_pos = T; p.mask = mask;

    bf16_t *kp = (bf16_t *)malloc(sizeof(bf16_t) * (size_t)Hkv * T * D);
    bf16_t *qp = (bf16_t *)malloc(sizeof(bf16_t) * (size_t)(rows ? rows : 1) * Hq * D);
    EXPECT(oracle_prepare_keys(&p, kp) == 0);
    EXPECT(oracle_prepare_queries(&p, qp) == 0);
    p.kp = kp;
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(rows ? rows : 1));
    for (int i = 0; i < rows; ++i)
        idx[i] = i;
    bf16_t *out = (bf16_t *)malloc(sizeof(bf16_t) * (size_t)(rows ? rows : 1) * Hq * D);
    bf16_t *ctx = (bf16_t *)malloc(sizeof(bf16_t) * (size_t)(rows ? rows : 1) * Hq * D);
    float *wsum = (float *)malloc(sizeof(float) * (size_t)(rows ? rows : 1) * Hq);
    float *wts = (float *)malloc(sizeof(float) * (size_t)(rows ? rows : 1) * Hq * T);
    EXPECT(oracle_attention(&p, idx, rows, out, ctx, wsum, wts) == 0);
    EXPECT(oracle_attention(&p, idx, rows, out, NULL, NULL, NULL) == 0);
    if (masked) {
        for (int h = 0; h < Hq; ++h)
            EXPECT(wsum[h] == 0.0f);                  /* the row with no visible key */
    }
    /* refusals */
    int32_t bad = rows;
    EXPECT(oracle_attention(&p, &bad, 1, out, NULL, NULL, NULL) == -1);
    bad = -1;
    EXPECT(oracle_attention(&p, &bad, 1, out, NULL, NULL, NULL) == -1);
    p.n_pos = T - 1;
    if (T > 0) {
        EXPECT(oracle_prepare_keys(&p, kp) == -1);
        EXPECT(oracle_prepare_queries(&p, qp) == -1);
        EXPECT(oracle_attention(&p, idx, rows, out, NULL, NULL, NULL) == -1);
    }
    p.n_pos = T;
    p.n_q_heads = Hq + 1;
    if ((Hq + 1) % Hkv != 0)
        EXPECT(oracle_attention(&p, idx, 0, out, NULL, NULL, NULL) == -1);
    p.n_q_heads = Hq;
    p.kp = NULL;
    EXPECT(oracle_attention(&p, idx, rows, out, NULL, NULL, NULL) == -1);
    free(qg); free(k); free(v); free(wq); free(wk); free(ct); free(st); free(mask);
    free(kp); free(qp); free(idx); free(out); free(ctx); free(wsum); free(wts);
}

int main(void)
{
    run_case(1, 2, 1, 0, 0, 1);
    run_case(37, 6, 2, 0, 0, 1);
    run_case(48, 4, 4, 16, 0, 1);
    run_case(40, 8, 2, 0, 1, 1);
    run_case(20, 4, 2, 0, 0, 0);
    run_case(33, 32, 2, 0, 0, 1);
    /* primitives: rounding of special values; a norm without rotary dims */
    const float sp[] = {0.0f, -0.0f, 1.0f, -1.0f, 3.3895314e38f, 1e-40f, -1e-45f, INFINITY, -INFINITY, NAN};
    bf16_t r[10];
    oracle_bf16_round(sp, r, 10);
    EXPECT(r[7] == 0x7f80 && r[8] == 0xff80 && (r[9] & 0x7f80) == 0x7f80 && (r[9] & 0x7f) != 0);
    bf16_t *x = bf16_buf(256, 1.0f), *w = bf16_buf(256, 0.1f), o[256];
    const float one = 1.0f, zero = 0.0f;
    oracle_norm_rope(x, w, &one, &zero, 256, 0, 1e-6f, o);
    free(x);
    free(w);
    EXPECT(oracle_abi() == 3 && oracle_mutation() == 0);
    printf("%s (%d failures)\n", failures ? "FAILED" : "oracle checks ok", failures);
    return failures ? 1 : 0;
}
